// Fused attention forward for gfx950 (CDNA4): MFMA + LDS-tiled online softmax.
//
// One workgroup of NW waves (NW = 4 or 8) owns a tile of BM = 32*NW query rows
// of one (sequence, head); wave w owns rows 32w..32w+31 of the tile. The kernel
// streams the visible keys in tiles of BN rows (64; 128 for D = 64, 4 waves) through a
// two-stage LDS ring (three stages for the 8-wave D = 128 plain instances, whose two
// wave groups run the tile chain half a tile apart) and, per tile, runs the fused
// chain of mlqm.cn/news/343191 §3.1
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
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernel.h"
#include "gfx950_util.h"

namespace sdpa08 {

constexpr int HEAD_GROUP = 4; // heads whose query tiles are interleaved on one XCD
constexpr float LAZY_RESCALE_LOG2 = 8.0f;
constexpr float OPT_LIMIT = 32768.0f;   // largest probability the optimistic pass accepts (fp16-safe)

// Softmax schemes of one key tile (see compute_tile).
constexpr int TILE_OPT = 0, TILE_MAX = 1, TILE_FAST = 2, TILE_FIRST = 3;
template <bool B> struct BoolTag { static constexpr bool value = B; };
template <int M> struct ModeTag { static constexpr int value = M; };

// MFMA order of one matrix phase of the ping-pong schedule (see the kernel):
// MODE PP_FULL runs P V of the previous tile and Q K^T of this one, the first AH
// MFMAs P V (their V operands are read before the barrier that opens the
// phase), then Q K^T and P V alternating, then the rest of Q K^T (so that no
// accumulation chain waits on its own previous result); PP_QK and PP_PV run one
// product alone. kind(n): 0 = P V, 1 = Q K^T; idx(n): which MFMA of that product.
constexpr int PP_FULL = 0, PP_QK = 1, PP_PV = 2;
template <int MODE, int AH, int NPV, int NQK> struct PPOrder {
  static constexpr int total = MODE == PP_FULL ? NPV + NQK : (MODE == PP_QK ? NQK : NPV);
  static constexpr int kind(int n) {
    if (MODE != PP_FULL) return MODE == PP_QK ? 1 : 0;
    if (n < AH) return 0;
    const int r = n - AH, pl = NPV - AH;
    return (r < 2 * pl && (r & 1)) ? 0 : 1;
  }
  static constexpr int idx(int n) {
    if (MODE != PP_FULL || n < AH) return n;
    const int r = n - AH, pl = NPV - AH;
    if (r < 2 * pl) return (r & 1) ? AH + (r >> 1) : (r >> 1);
    return pl + (r - 2 * pl);
  }
  static constexpr int reads(int n) { return kind(n) == 0 ? 2 : 1; }   // LDS reads of operand A
  static constexpr int reads_before(int n) { return n <= 0 ? 0 : reads(n - 1) + reads_before(n - 1); }
};
// Scheduling groups of a matrix phase: before MFMA n, the reads of MFMA n + AH.
template <class O, int AH, int N> __device__ __forceinline__ void pp_groups() {
  if constexpr (N < O::total) {
    if constexpr (N + AH < O::total) __builtin_amdgcn_sched_group_barrier(0x100, O::reads(N + AH), 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    pp_groups<O, AH, N + 1>();
  }
}

// One stage of an LDS ring: where a key tile's K rows and V rows go.
struct Stage { uint8_t* k; uint8_t* v; };

// acc + lo(p) + hi(p) for a pair of fp16 values (one v_dot2).
__device__ __forceinline__ float add_pair_f16(uint32_t p, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), one, acc, false);
}

// KS = 2: the waves form two groups that share the workgroup's query rows and
// take alternate key blocks of every tile; the two partial results (running
// maximum, row sum, accumulator) are merged through LDS at the end. It doubles
// the waves per query tile, so problems with few tiles fill the chip in whole
// rounds instead of leaving a half-empty last round.
//
// AB: the ALiBi bias alone (no window, no global rows) on the ping-pong
// schedule; the other mask variants take EXT (4 waves).
template <int D, bool BF16, bool CAUSAL, bool VARLEN, int NW, bool EXT, int KS, bool AB = false>
__global__ __launch_bounds__(NW * 64, (D == 64 && NW == 4 && !EXT) ? 3 : 8 / NW) void attn_fwd_kernel(FwdParams p) {
  constexpr int NWAVES = NW;
  constexpr int NWR = NW / KS;                 // waves per key group (one per 32 query rows)
  constexpr int BM = 32 * NWR;                 // query rows per workgroup
  // Keys per group block: 128 for D = 64 with 4 waves per group (the same
  // 16 KB as 64 keys of D = 128, twice the matrix work per barrier and per
  // softmax pass; measured 2-7 % faster on B4 H12 S2048, 7 % slower with 8
  // waves on 256 rows), else 64.
  constexpr int BN = 64;
  constexpr int GBN = KS * BN;                 // keys per LDS tile (all groups)
  constexpr int NKB = BN / 32;                 // 32-key blocks per group block
  constexpr int ROWB = D * 2;                  // bytes per K/V row
  constexpr int TILEB = BN * ROWB;             // bytes of one group's K (or V) block
  constexpr int GTILEB = GBN * ROWB;           // bytes per K (or V) tile
  constexpr int STAGEB = 2 * GTILEB;           // K tile + V tile
  constexpr int LDW = GTILEB / 1024 / NWAVES;  // 1 KB direct loads per wave per tile
  static_assert(KS == 1 || (KS == 2 && !EXT), "key split: plain masks only");
  constexpr int DCH = D / 16;                  // 16-deep contraction chunks of Q K^T
  constexpr int DB = D / 32;                   // 32-row blocks of O^T
  static_assert(LDW >= 1, "tile must give every wave a 1 KB load");

  // Two separate arrays, one per stage: the compiler can then tell that LDS
  // reads of one stage never alias the in-flight direct loads into the other
  // and does not wait for those loads before every read.
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[STAGEB];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[STAGEB];
  __shared__ int redo_flag;     // some wave saw a probability above OPT_LIMIT
  // The three-stage ring of the ping-pong instances keeps K and V tiles in
  // arrays of their own, the K tiles below 48 KB and the V tiles above: every
  // read of either kind then reaches all three stages from one register of lane
  // offsets plus the instruction's 16-bit immediate offset (with 32 KB stages the
  // third one starts at 64 KB, past that offset, and its reads needed address
  // arithmetic and registers of their own).
  __shared__ __attribute__((aligned(1024))) uint8_t pk0[GTILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t pk1[GTILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t pk2[GTILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t pv0[GTILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t pv1[GTILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t pv2[GTILEB];
  // The 8-wave D = 128 plain instances run the ping-pong schedule (below) on a
  // three-stage ring.
  constexpr bool PINGPONG = !EXT && KS == 1 && NW == 8 && D == 128;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Ping-pong instances: wave-uniform, so that the LDS addresses of the direct
  // loads are scalar. (In the D = 64 8-wave instances the scalar form raised
  // the registers from 126 to 154, past two workgroups per CU.)
  const int wave = PINGPONG ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int li = lane & 31;     // query row inside the wave / MFMA row index
  const int hh = lane >> 5;     // which half of the contraction this lane feeds
  const int wr = KS == 1 ? wave : wave % NWR;   // which 32 query rows of the tile
  const int kgrp = KS == 1 ? 0 : wave / NWR;    // which key block of every tile

  // ---- which (sequence, head, query tile) this workgroup owns -------------
  // Workgroup i runs on XCD i % 8. Undo that interleave so each XCD owns a
  // contiguous run of the logical order, then walk heads in groups of
  // HEAD_GROUP with the query tiles of a group interleaved, longest (causal)
  // tiles first. An XCD then works on a few heads at a time, whose K/V stay
  // in its L2, and the longest tiles start first.
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int nbh = VARLEN ? p.H : p.B * p.H;
  const int nt = p.n_qtiles;
  // Heads per group: chosen by the launcher.
  const int HGRP = p.head_group;
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
  const int j_lo = kv_lo / GBN;
  const int n_kv = (kv_hi + GBN - 1) / GBN;        // one past the last tile
  const int wq0 = q0 + wr * 32;          // first query row of this wave
  const int qi = wq0 + li;               // this lane's query row
  // Mask-variant state of this wave (EXT only).
  const int win = EXT ? p.window : 0;
  const int n_glob = EXT ? p.n_global : 0;
  const bool w_any_glob = EXT && wq0 < n_glob;          // some row of the wave is global
  const bool w_all_glob = EXT && wq0 + 31 < n_glob;     // every row of the wave is global
  const float slope2 = ((EXT || AB) && p.alibi != nullptr) ? p.alibi[h] * 1.4426950408889634f : 0.0f;
  const bool use_alibi = AB || (EXT && p.alibi != nullptr);
  const uint32_t q_rows = (uint32_t)min(L - q0, BM);

  // ---- Q^T operand, resident in registers for the whole key loop ----------
  // Rows past the sequence end read as zeros (buffer range check).
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(qg, q_rows * tok_bytes);
  const uint32_t q_voff = (uint32_t)(wr * 32 + li) * tok_bytes + hh * 16;
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
  // Ping-pong instances: the V stages lie above 48 KB (see the arrays); the lane
  // offsets carry that bias so that every V read is register + immediate offset.
  constexpr int VBIAS = PINGPONG ? 3 * GTILEB : 0;
  uint32_t v_off[2][DB];
  {
    const int blk = li >> 4, s = li & 15;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int key = t2 * 8 + hh * 4 + (s >> 2);        // + 16 * (16-key step)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = db * 32 + blk * 16 + swap23(4 * (s & 3));
        v_off[t2][db] = key * ROWB + ((((col >> 3) ^ swz<D>(key)) << 4) | ((col & 7) * 2)) + VBIAS;
        // Ping-pong: the bias must stay in the register (the compiler would fold it
        // back into the stage address, past the immediate-offset range).
        if constexpr (PINGPONG) asm volatile("" : "+v"(v_off[t2][db]));
      }
    }
  }

  // The ring's stages (the ping-pong instances: three, in the arrays above).
  const Stage st0 = PINGPONG ? Stage{pk0, pv0} : Stage{smem0, smem0 + GTILEB};
  const Stage st1 = PINGPONG ? Stage{pk1, pv1} : Stage{smem1, smem1 + GTILEB};
  const Stage st2 = {pk2, pv2};

  // Issue the direct loads of key tile j into `stage` (K tile, then V tile).
  auto issue_to = [&](int j, const Stage& stage) {
    const int key0 = j * GBN;
    const uint32_t rows = (uint32_t)min(L - key0, GBN);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kg + (size_t)key0 * p.H * D, rows * tok_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vg + (size_t)key0 * p.H * D, rows * tok_bytes);
    uint8_t* kdst = stage.k + wave * LDW * 1024;
    uint8_t* vdst = stage.v + wave * LDW * 1024;
#pragma unroll
    for (int u = 0; u < LDW; ++u) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kdst + u * 1024), 16, (int)ld_voff[u], 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < LDW; ++u) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vdst + u * 1024), 16, (int)ld_voff[u], 0, 0, 0);
    }
  };
  auto issue_tile = [&](int j, int st) { issue_to(j, st ? st1 : st0); };

  // ---- running statistics and accumulator --------------------------------
  f32x16 acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = f32x16{};
  float m_run = -INFINITY;     // running max of the log2-scaled logits
  float l_run = 0.0f;          // this lane's half of the running exp-sum
  uint64_t bad = 0;            // TILE_FAST: lanes whose tile sum failed the bound
  // The plain instances (no mask variant, no key split) walk their tiles after
  // the first with TILE_FAST: every row sees key 0 of its first tile, so the
  // first tile's row maximum is finite and serves as the reference for the rest.
  constexpr bool FAST_LOOP = !EXT && KS == 1;

  // ALiBi in the log2-scaled domain: t = s * c - slope * |i - j| for the scores
  // of a tile starting at key key0. slope * (j - i) = slope * (key0 + 4 hh - i)
  // + slope * (offset of the register), and -|x| = min(x, -x).
  auto alibi_bias = [&](f32x16 (&sv)[NKB], int key0) __attribute__((always_inline)) {
    const float bl = slope2 * (float)(key0 + hh * 4 - qi);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float u = fmaf(slope2, (float)(kb * 32 + (r >> 2) * 8 + (r & 3)), bl);
        sv[kb][r] = fmaf(sv[kb][r], c_log2, fminf(u, -u));
      }
    }
  };

  // One key tile. MASKED (compile time): the tile may hold keys some row of the
  // workgroup must not see (diagonal, sequence end, mask variants); without it
  // the mask code is left out. MODE (compile time) picks the softmax scheme:
  //   TILE_OPT:  optimistic exponentials, checked on the spot (redone against a
  //              refreshed maximum when the check fails);
  //   TILE_MAX:  the tile's row maximum first, then the exponentials;
  //   TILE_FAST: optimistic exponentials against the running maximum with no
  //              branch between them and P V; the check only raises `bad`,
  //              which the workgroup acts on after its last tile;
  //   TILE_FIRST: a wave's first tile when each of its rows sees a key of it:
  //              the row maximum becomes the running maximum (the accumulator
  //              and the sum are still zero), again with no branch.
  auto compute_tile = [&](auto masked_c, auto mode_c, int j, const Stage& stage) {
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr int MODE = decltype(mode_c)::value;
    const uint8_t* ks = stage.k + kgrp * TILEB;
    const uint8_t* vs = stage.v + kgrp * TILEB;
    const int key0 = j * GBN + kgrp * BN;
    // A wave none of whose rows sees a key of this tile has nothing to do.
    if constexpr (MASKED) {
      if constexpr (EXT) {
        if (!w_any_glob) {
          if (CAUSAL && key0 > wq0 + 31) return;
          if (win > 0 && key0 + BN - 1 <= wq0 - win) return;
          if (win > 0 && !CAUSAL && key0 >= wq0 + 31 + win) return;
        }
      } else {
        if (CAUSAL && key0 > wq0 + 31) return;
      }
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
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NKB, 0);
#pragma unroll
      for (int c = 0; c < DCH; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, NKB, 0);
        if (c + 2 < DCH) __builtin_amdgcn_sched_group_barrier(0x100, NKB, 0);
      }
    }

    // Mask keys past the sequence end and, under causality, keys after the
    // query (only tiles that reach those positions pay for it).
    bool need_mask = MASKED && ((key0 + BN > L) || (CAUSAL && key0 + BN - 1 > wq0));
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
        alibi_bias(s, key0);
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
    } else {
      if constexpr (AB) alibi_bias(s, key0);
      if (need_mask) {
        // Register r of block kb holds key key0 + 4 hh + c, c = 32 kb + 8 (r / 4) + r % 4
        // (a constant): visible iff key < L and, causal, key <= qi, i.e. c <= T.
        const int T = (CAUSAL ? min(L - 1, qi) : L - 1) - key0 - hh * 4;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
            s[kb][r] = c <= T ? s[kb][r] : -INFINITY;
          }
        }
      }
    }

    // With ALiBi the scores are already log2-scaled.
    const bool prescaled = (EXT || AB) && use_alibi;
    const float c_mul = prescaled ? 1.0f : c_log2;
    // P = exp2(s * c - m), packed to 16 bit for P V; returns this lane's half
    // of the tile's row sum.
    // l: bf16 keeps 8 significant bits, so a row with few visible keys would
    // carry up to 2^-9 relative error into ln(l) if l summed the rounded
    // values; it sums the fp32 values instead. fp16 (11 bits) keeps that
    // error below 2.5e-4 and sums the rounded pairs with one dot2.
    uint32_t pk[NKB][8];
    auto exps = [&](float m_sub) {
      float tl = BF16 ? -0.0f : 0.0f;   // -0 + x folds to x (bf16 sums fp32 adds)
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
    bool redo = MODE == TILE_OPT || MODE == TILE_MAX;
    if constexpr (MODE == TILE_FIRST) {
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      }
      m_run = half_max(mx) * c_log2;
      tile_l = exps(m_run);
    } else if constexpr (MODE == TILE_FAST) {
      tile_l = exps(m_run);
      bad |= __builtin_amdgcn_ballot_w64(!(tile_l <= OPT_LIMIT));
    } else if (MODE == TILE_OPT && j != j_lo) {
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
      // are all -inf too): subtract 0 instead, which gives exp2(-inf) = 0. (Only
      // with the mask variants or the key split can a wave's first tile hold
      // rows that see none of its keys.)
      tile_l = exps(((EXT || KS > 1) && m_run == -INFINITY) ? 0.0f : m_run);
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
        const uint8_t* vb = vs - VBIAS + kc * 16 * ROWB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + v_off[0][d]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + v_off[1][d]));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 a = {lo2[0], lo2[1], hi2[0], hi2[1]};
        acc[d] = mfma32<BF16>(a, bop, acc[d]);
      }
    }
  };

  // ---- main loop ---------------------------------------------------------------
  constexpr BoolTag<true> masked_t{};
  constexpr BoolTag<false> plain_t{};
  if (tid == 0) redo_flag = 0;
  issue_tile(j_lo, 0);
  wait_vmem_all();
  __syncthreads();
  if constexpr (!FAST_LOOP) {
#pragma unroll 1
    for (int j = j_lo; j < n_kv; j += 2) {
      if (j + 1 < n_kv) issue_tile(j + 1, 1);
      compute_tile(masked_t, ModeTag<TILE_OPT>{}, j, st0);
      wait_vmem_all();
      __syncthreads();
      if (j + 1 >= n_kv) break;
      if (j + 2 < n_kv) issue_tile(j + 2, 0);
      compute_tile(masked_t, ModeTag<TILE_OPT>{}, j + 1, st1);
      wait_vmem_all();
      __syncthreads();
    }
  } else {
    if constexpr (PINGPONG) {
      // Ping-pong schedule. Waves w and w + 4 share a SIMD. Each wave alternates
      // a matrix phase M(t) (P V of tile t-1, then Q K^T of tile t) and a vector
      // phase S(t) (the softmax of tile t), with a workgroup barrier after every
      // phase; waves 4-7 run one phase behind waves 0-3, so on every SIMD one
      // wave's MFMAs overlap the other's exponentials instead of both waves
      // entering the same phase together. A single wave keeps the matrix core
      // fed only if its LDS operands are read well ahead: each MFMA's operand is
      // read PP_AH MFMAs before it, and the first PP_AH (V operands) before the
      // barrier that opens the phase.
      //   Phase p:   0     1     2     3     ...  2t    2t+1  ...  2n    2n+1
      //   waves 0-3: M(0)  S(0)  M(1)  S(1)       M(t)  S(t)       M(n)
      //   waves 4-7: -     M(0)  S(0)  M(1)       S(t-1) M(t)      S(n-1) M(n)
      // Tile t sits in stage t % 3. Its loads go out at the start of phase 2t-2
      // (when the stage's previous tile, t-3, was last read: its V in phase
      // 2t-3) and are waited for at the end of phase 2t-1, so the Q K^T of
      // phase 2t and the V reads issued during phase 2t+1 find them in LDS.
      // Waits come only at the end of odd phases; the other barriers are bare
      // (a __syncthreads() would also wait for the loads in flight and for the
      // reads issued ahead of the next phase).
      constexpr int NPV = 2 * NKB * DB;     // P V MFMAs per tile and wave
      constexpr int NQK = DCH * NKB;        // Q K^T MFMAs per tile and wave
      constexpr int PP_AH = 4;              // operand reads ahead of their MFMA
      f32x16 sc[NKB];                       // scores of the tile whose softmax is next
      uint32_t pk[NKB][8];                  // its probabilities, 16 bit
      u32x4 ab[NPV + NQK];                  // operand A of each MFMA of a matrix phase

      // Wait for this wave's loads at the end of a phase (nothing moves across it).
      auto pp_wait = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        wait_vmem_all();
      };
      auto pp_bar = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      };
      // Operand A of MFMA n of a matrix phase: V^T of 16 keys by two transposing
      // reads, or a 32-key block of K.
      auto rd = [&](auto mode_c, int n, const uint8_t* vs, const uint8_t* ks) __attribute__((always_inline)) {
        using O = PPOrder<decltype(mode_c)::value, PP_AH, NPV, NQK>;
        const int i = O::idx(n);
        if (O::kind(n) == 0) {
          const int kc = i / DB, d = i % DB;
          const uint8_t* vb = vs - VBIAS + kc * 16 * ROWB;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + v_off[0][d]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + v_off[1][d]));
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
        }
        const int c = i / NKB, kb = i % NKB;
        return *reinterpret_cast<const u32x4*>(ks + kb * 32 * ROWB + k_off[c]);
      };
      // Reads of the first PP_AH operands of the next matrix phase (all V).
      auto m_pre = [&](const Stage& vstage) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < PP_AH; ++n) ab[n] = rd(ModeTag<PP_FULL>{}, n, vstage.v, nullptr);
      };
      // Matrix phase: P V from `vstage` with pk, then / interleaved with
      // S^T = K Q^T from `kstage` into sc. PIN: the first reads are issued here.
      auto m_phase = [&](auto mode_c, auto pin_c, const Stage& vstage, const Stage& kstage)
          __attribute__((always_inline)) {
        using O = PPOrder<decltype(mode_c)::value, PP_AH, NPV, NQK>;
        constexpr bool PIN = decltype(pin_c)::value;
        const uint8_t* vs = vstage.v;
        const uint8_t* ks = kstage.k;
        if constexpr (PIN) {
#pragma unroll
          for (int n = 0; n < PP_AH; ++n) ab[n] = rd(mode_c, n, vs, ks);
        }
#pragma unroll
        for (int n = 0; n < O::total; ++n) {
          if (n + PP_AH < O::total) ab[n + PP_AH] = rd(mode_c, n + PP_AH, vs, ks);
          const int i = O::idx(n);
          if (O::kind(n) == 0) {
            const int kc = i / DB, d = i % DB, kb = kc >> 1, e = kc & 1;
            const u32x4 bop = {pk[kb][e * 4 + 0], pk[kb][e * 4 + 1], pk[kb][e * 4 + 2], pk[kb][e * 4 + 3]};
            acc[d] = mfma32<BF16>(ab[n], bop, acc[d]);
          } else {
            const int c = i / NKB, kb = i % NKB;
            sc[kb] = mfma32<BF16>(ab[n], qreg[c], c == 0 ? f32x16{} : sc[kb]);
          }
        }
        if constexpr (PIN) __builtin_amdgcn_sched_group_barrier(0x100, O::reads_before(PP_AH), 0);
        pp_groups<O, PP_AH, 0>();
      };
      // Vector phase: mask (diagonal and tail tiles), exponentials, row sums.
      auto s_phase = [&](auto masked_c, auto first_c, int j) __attribute__((always_inline)) {
        const int key0 = j * GBN;
        if constexpr (decltype(masked_c)::value) {
          if ((key0 + BN > L) || (CAUSAL && key0 + BN - 1 > wq0)) {
            // key key0 + 4 hh + c is visible iff c <= T (as in compute_tile)
            const int T = (CAUSAL ? min(L - 1, qi) : L - 1) - key0 - hh * 4;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
                sc[kb][r] = c <= T ? sc[kb][r] : -INFINITY;
              }
            }
          }
        }
        if constexpr (decltype(first_c)::value) {
          // every row sees key 0 of its first tile: the maximum is finite. With
          // ALiBi it is taken over the unbiased scores: the bias is never
          // positive and is zero at the row's own key, so this bounds every
          // biased score of the tile, and later tiles (whose scores rise toward
          // the diagonal only through the bias) stay within the optimistic bound
          // as often as without it.
          float mx = sc[0][0];
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
          }
          m_run = half_max(mx) * c_log2;
        }
        if constexpr (AB && !CAUSAL) alibi_bias(sc, key0);      // scores now log2-scaled
        // Under causality every key a row sees has j <= i, so its bias is
        // slope * (j - i) with no absolute value, and the running maximum folds
        // into the per-lane base: each exponent then takes two fused
        // multiply-adds (masked scores stay -inf).
        const float bm = (AB && CAUSAL) ? fmaf(slope2, (float)(key0 + hh * 4 - qi), -m_run) : 0.0f;
        auto expo = [&](int kb, int r) __attribute__((always_inline)) {
          if constexpr (AB && CAUSAL) {
            const float w = fmaf(slope2, (float)(kb * 32 + (r >> 2) * 8 + (r & 3)), bm);
            return __builtin_amdgcn_exp2f(fmaf(sc[kb][r], c_log2, w));
          } else if constexpr (AB) {
            return __builtin_amdgcn_exp2f(sc[kb][r] - m_run);
          } else {
            return __builtin_amdgcn_exp2f(fmaf(sc[kb][r], c_log2, -m_run));
          }
        };
        float tl = BF16 ? -0.0f : 0.0f;   // -0 + x folds to x (bf16 sums fp32 adds)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float e0 = expo(kb, 2 * t);
            const float e1 = expo(kb, 2 * t + 1);
            pk[kb][t] = pack2<BF16>(e0, e1);
            if constexpr (BF16) {
              tl += e0 + e1;
            } else {
              tl = add_pair_f16(pk[kb][t], tl);
            }
          }
        }
        if constexpr (!decltype(first_c)::value) bad |= __builtin_amdgcn_ballot_w64(!(tl <= OPT_LIMIT));
        l_run += tl;
        // Keep the packing in this phase (the compiler would sink it to the P V
        // MFMAs, into the matrix phase).
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int t = 0; t < 8; ++t) asm volatile("" : "+v"(pk[kb][t]));
        }
      };
      const int n = n_kv - j_lo;            // tiles of this workgroup (>= 1)
      // Tiles [0, n_pl) need no mask. Plain steps t = 1 .. t_pe - 1 (a multiple of
      // three of them, so the masked loop starts on the same stage rotation), all
      // before the last step.
      int n_pl = min(n_kv, L / GBN);
      if (CAUSAL) n_pl = min(n_pl, (q0 + 1) / GBN);
      n_pl -= j_lo;
      const int t_pe = 1 + max(0, min(n_pl, n - 1) - 1) / 3 * 3;

      // The schedule is compiled once per wave group, so that no branch on the
      // group sits between a load and its wait (the compiler would then assume
      // the other group's loads in flight and wait for them before LDS reads).
      auto schedule = [&](auto late_c) __attribute__((always_inline)) {
        constexpr bool LATE = decltype(late_c)::value;
        // One step: S(t), then M(t+1) (LAST: P V of tile t alone, no barrier after
        // it for waves 4-7, whose last phase it is). Stages: V of tile t in vst,
        // K of tile t+1 in kst, tile t+2 goes into ist.
        auto step = [&](auto masked_c, auto first_c, auto last_c, int t, const Stage& vst,
                        const Stage& kst, const Stage& ist) __attribute__((always_inline)) {
          constexpr bool LAST = decltype(last_c)::value;
          constexpr bool SKIP = decltype(masked_c)::value && CAUSAL;
          const int j = j_lo + t;
          // Under causality a wave none of whose rows sees a key of tile t skips
          // the softmax of tile t, the P V of tile t and the Q K^T of tile t+1 (and
          // every later phase; the Q K^T of the first tile it does not see is still
          // computed): its scores there are all masked, so they would add nothing.
          // It still takes every barrier.
          const bool act0 = !(SKIP && j * GBN > wq0 + 31);
          if (!LAST && LATE && t + 2 < n) issue_to(j + 2, ist);     // phase 2t+2 of waves 4-7
          if (act0) {
            s_phase(masked_c, first_c, j);
            m_pre(vst);
          }
          if constexpr (!LATE) pp_wait();                           // end of phase 2t+1
          pp_bar();
          if (!LAST && !LATE && t + 2 < n) issue_to(j + 2, ist);    // phase 2t+2 of waves 0-3
          if (act0) {
            if constexpr (LAST) {
              m_phase(ModeTag<PP_PV>{}, BoolTag<false>{}, vst, vst);
            } else {
              m_phase(ModeTag<PP_FULL>{}, BoolTag<false>{}, vst, kst);
            }
          }
          if constexpr (LATE) pp_wait();                            // end of phase 2t+3
          if constexpr (!LAST || !LATE) pp_bar();
        };
        // Phase 0 (1 for waves 4-7): Q K^T of tile 0, whose loads the barrier
        // above waited for; tile 1 goes out at the start of phase 0.
        if (n > 1) issue_to(j_lo + 1, st1);
        if constexpr (LATE) pp_bar();
        m_phase(ModeTag<PP_QK>{}, BoolTag<true>{}, st0, st0);
        if constexpr (LATE) pp_wait();
        pp_bar();
        if (n == 1) {
          step(masked_t, BoolTag<true>{}, BoolTag<true>{}, 0, st0, st0, st0);
        } else {
          step(masked_t, BoolTag<true>{}, BoolTag<false>{}, 0, st0, st1, st2);
#pragma unroll 1
          for (int t = 1; t < t_pe; t += 3) {
            step(plain_t, BoolTag<false>{}, BoolTag<false>{}, t, st1, st2, st0);
            step(plain_t, BoolTag<false>{}, BoolTag<false>{}, t + 1, st2, st0, st1);
            step(plain_t, BoolTag<false>{}, BoolTag<false>{}, t + 2, st0, st1, st2);
          }
#pragma unroll 1
          for (int t = t_pe; t < n - 1; t += 3) {
            step(masked_t, BoolTag<false>{}, BoolTag<false>{}, t, st1, st2, st0);
            if (t + 1 >= n - 1) break;
            step(masked_t, BoolTag<false>{}, BoolTag<false>{}, t + 1, st2, st0, st1);
            if (t + 2 >= n - 1) break;
            step(masked_t, BoolTag<false>{}, BoolTag<false>{}, t + 2, st0, st1, st2);
          }
          // The last step: no loads are in flight any more, so its stage may be
          // chosen at run time.
          const int sl = (n - 1) % 3;
          const Stage vl = sl == 0 ? st0 : (sl == 1 ? st1 : st2);
          step(masked_t, BoolTag<false>{}, BoolTag<true>{}, n - 1, vl, vl, vl);
        }
      };
      if (wave >= 4) {
        schedule(BoolTag<true>{});
      } else {
        schedule(BoolTag<false>{});
      }
    } else {
      // Tiles before j_plain hold no key that any row of the workgroup must not
      // see: they run without the mask code, in a loop of their own (a branch
      // between the two kinds inside one loop makes the compiler copy the
      // accumulators at every join). Their count after the first tile is kept
      // even so that the masked loop always starts on stage 1.
      int j_plain = min(n_kv, L / GBN);
      if (CAUSAL) j_plain = min(j_plain, (q0 + 1) / GBN);
      j_plain = j_lo + 1 + (max(0, j_plain - (j_lo + 1)) & ~1);
      // First tile: row maxima, the reference of the optimistic tiles after it.
      if (j_lo + 1 < n_kv) issue_tile(j_lo + 1, 1);
      compute_tile(masked_t, ModeTag<TILE_FIRST>{}, j_lo, st0);
      wait_vmem_all();
      __syncthreads();
#pragma unroll 1
      for (int j = j_lo + 1; j < j_plain; j += 2) {
        issue_tile(j + 1, 0);
        compute_tile(plain_t, ModeTag<TILE_FAST>{}, j, st1);
        wait_vmem_all();
        __syncthreads();
        if (j + 2 < n_kv) issue_tile(j + 2, 1);
        compute_tile(plain_t, ModeTag<TILE_FAST>{}, j + 1, st0);
        wait_vmem_all();
        __syncthreads();
      }
#pragma unroll 1
      for (int j = j_plain; j < n_kv; j += 2) {
        if (j + 1 < n_kv) issue_tile(j + 1, 0);
        compute_tile(masked_t, ModeTag<TILE_FAST>{}, j, st1);
        wait_vmem_all();
        __syncthreads();
        if (j + 1 >= n_kv) break;
        if (j + 2 < n_kv) issue_tile(j + 2, 1);
        compute_tile(masked_t, ModeTag<TILE_FAST>{}, j + 1, st0);
        wait_vmem_all();
        __syncthreads();
      }
    }
    // Some tile of some wave exceeded the bound (its maximum grew by more than
    // log2(OPT_LIMIT) over the first tile's): the whole workgroup walks its keys
    // again from scratch, every tile's row maximum first. Every load has landed
    // and every wave is past its last barrier, so the ring is free.
    if (bad != 0 && lane == 0) redo_flag = 1;
    __syncthreads();
    if (redo_flag != 0) {
#pragma unroll
      for (int d = 0; d < DB; ++d) acc[d] = f32x16{};
      m_run = -INFINITY;
      l_run = 0.0f;
#pragma unroll 1
      for (int j = j_lo; j < n_kv; ++j) {
        issue_tile(j, 0);
        wait_vmem_all();
        __syncthreads();
        compute_tile(masked_t, ModeTag<TILE_MAX>{}, j, st0);
        __syncthreads();
      }
    }
  }

  if constexpr (KS == 2) {
    // Merge the two key groups through LDS (the loop ended with every load
    // done and every wave past its last barrier, so both stages are free).
    // Group 0 saw key 0 of every row, so its running maximum is finite.
    float* xa = reinterpret_cast<float*>(smem0);   // [NWR][DB][16][64] accumulators
    float* xm = reinterpret_cast<float*>(smem1);   // [NWR][2][64] maximum and row sum
    static_assert(NWR * DB * 16 * 64 * 4 <= STAGEB, "merge area");
    if (kgrp == 1) {
#pragma unroll
      for (int d = 0; d < DB; ++d) {
#pragma unroll
        for (int r = 0; r < 16; ++r) xa[((wr * DB + d) * 16 + r) * 64 + lane] = acc[d][r];
      }
      xm[(wr * 2 + 0) * 64 + lane] = m_run;
      xm[(wr * 2 + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    if (kgrp == 1) return;
    const float m1 = xm[(wr * 2 + 0) * 64 + lane];
    const float l1 = xm[(wr * 2 + 1) * 64 + lane];
    const float mm = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - mm);
    const float a1 = (m1 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[d][r] = fmaf(acc[d][r], a0, xa[((wr * DB + d) * 16 + r) * 64 + lane] * a1);
      }
    }
    l_run = fmaf(l_run, a0, l1 * a1);
    m_run = mm;
  }

  // ---- epilogue: O = acc / l, LSE = ln(l) + m -------------------------------
  const float l_tot = half_sum(l_run);
  const float inv = 1.0f / l_tot;
  // Stores past the sequence end fall outside the descriptor and are dropped.
  const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(og, q_rows * tok_bytes);
  const uint32_t o_voff = (uint32_t)(wr * 32 + li) * tok_bytes + hh * 16;
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


// Workgroup shape by problem size (query tiles of 256 rows, 128-row tiles
// counted per (batch, head) pair):
//  * 8 waves on 256 rows (one workgroup per CU) when there are enough 256-row
//    tiles to fill the chip several times over;
//  * 8 waves on 128 rows with the keys of every tile split between two wave
//    groups (KS = 2, one workgroup per CU) when the 128-row tiles fit in one
//    round of the 256 CUs: twice the waves per tile (B1 H8 S4096 D128 causal,
//    256 tiles: 55 us vs 71 us with 4 waves; B2 H4 S2048 D64, 128 tiles: 20 vs
//    24 us). With more tiles the 4-wave shape is faster (B4 H12 S2048 D64, 768
//    tiles: 60 vs 65 us; B1 H16 S8192 D128 causal, 1024 tiles: 255 vs 264 us);
//  * else 4 waves on 128 rows (two workgroups per CU).
constexpr long long kBigProblemTiles = 2048;
constexpr long long kKeySplitMaxTiles = 256;

enum class Shape { W4, W8, W8_KS2 };

static Shape choose_shape(const FwdParams& p, bool varlen, const FwdTuning& t) {
  if (t.tile_rows == 256) return Shape::W8;
  if (t.tile_rows == 128) return t.key_split == 2 ? Shape::W8_KS2 : Shape::W4;
  const long long bh = varlen ? p.H : (long long)p.B * p.H;
  const long long tiles256 = varlen ? (long long)p.S / 256 + p.B : ((long long)p.S + 255) / 256;
  const long long tiles128 = varlen ? (long long)p.S / 128 + p.B : ((long long)p.S + 127) / 128;
  if (tiles256 * bh >= kBigProblemTiles) return Shape::W8;
  if (t.key_split == 1) return Shape::W4;
  if (t.key_split == 2 || tiles128 * bh <= kKeySplitMaxTiles) return Shape::W8_KS2;
  return Shape::W4;
}

int max_query_tile_rows() { return 256; }
int min_query_tile_rows() { return 128; }

// Heads per XCD group for 128-row tiles. Each XCD owns a contiguous run of
// about nbh / 8 heads; when the K and V of that whole run fit in the XCD's
// 4 MB L2, one group spans it, so the XCD starts the longest causal tiles of
// all its heads first (B4 H12 S2048 D64: 6 heads of 0.5 MB, causal +11 % over
// groups of 2 and +17 % over 4, non-causal unchanged; groups of 8, which
// straddle XCDs, gained nothing). Otherwise groups of 2 (16 heads of 2 MB
// measured clearly slower).
static int head_group_128(const FwdParams& p, int D, bool varlen) {
  const long long nbh = varlen ? p.H : (long long)p.B * p.H;
  const long long per_xcd = (nbh + NXCD - 1) / NXCD;
  const long long kv_bytes_head = (long long)p.S * D * 2 * 2;   // K and V, 16-bit (S = T when packed)
  const long long l2_bytes = 4LL << 20;
  long long g = (per_xcd * kv_bytes_head <= l2_bytes) ? per_xcd : 2;
  if (g > nbh) g = nbh;
  return g < 1 ? 1 : (int)g;
}

// Heads per XCD group for 256-row tiles: HEAD_GROUP, except for long padded
// sequences whose K and V per head exceed 8 MB, where groups of 2 put more of
// an XCD's concurrent workgroups on one head's K/V stream (B1 H32 S65536 D64
// causal: 16.9 ms with groups of 2 or 1, 17.3 ms with 4, 22 ms with 8; the
// LLaMA-shaped layer and the packed batch are fastest with 4).
static int head_group_256(const FwdParams& p, int D, bool varlen) {
  const long long kv_bytes_head = (long long)p.S * D * 2 * 2;
  return (!varlen && kv_bytes_head > (8LL << 20)) ? 2 : HEAD_GROUP;
}

template <int D, bool BF16, bool CAUSAL, bool VARLEN, int NW, bool EXT, int KS, bool AB = false>
static hipError_t launch_one(FwdParams p, int head_group, hipStream_t stream) {
  constexpr long long BM = 32 * NW / KS;
  const long long tiles = VARLEN ? (long long)p.S / BM + p.B : ((long long)p.S + BM - 1) / BM;
  p.n_qtiles = (int)tiles;
  const long long nbh = VARLEN ? p.H : (long long)p.B * p.H;
  if (head_group <= 0) {
    head_group = EXT ? HEAD_GROUP : BM == 128 ? head_group_128(p, D, VARLEN)
                                              : head_group_256(p, D, VARLEN);
  }
  p.head_group = (int)(head_group < nbh ? head_group : nbh);
  const long long grid = tiles * nbh;
  hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, CAUSAL, VARLEN, NW, EXT, KS, AB>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool BF16, bool CAUSAL, bool VARLEN>
static hipError_t launch_nw(const FwdParams& p, const FwdTuning& t, hipStream_t stream) {
  // The mask/bias variants run with 4-wave workgroups, except ALiBi alone at
  // D = 128 where the plain instances would take 8 waves on 256 rows: it runs
  // on their ping-pong schedule (the bias adds 2 VALU per score to the softmax
  // phases, which still fit beside the other wave's matrix phase).
  if (p.window > 0 || p.n_global > 0 || p.alibi != nullptr) {
    if constexpr (D == 128) {
      if (p.window == 0 && p.n_global == 0 && choose_shape(p, VARLEN, t) == Shape::W8) {
        return launch_one<D, BF16, CAUSAL, VARLEN, 8, false, 1, true>(p, t.head_group, stream);
      }
    }
    return launch_one<D, BF16, CAUSAL, VARLEN, 4, true, 1>(p, t.head_group, stream);
  }
  switch (choose_shape(p, VARLEN, t)) {
    case Shape::W8: return launch_one<D, BF16, CAUSAL, VARLEN, 8, false, 1>(p, t.head_group, stream);
    case Shape::W8_KS2:
      return launch_one<D, BF16, CAUSAL, VARLEN, 8, false, 2>(p, t.head_group, stream);
    default: return launch_one<D, BF16, CAUSAL, VARLEN, 4, false, 1>(p, t.head_group, stream);
  }
}

template <int D, bool BF16>
static hipError_t launch_d(const FwdParams& p, const FwdTuning& t, bool causal, bool varlen,
                           hipStream_t stream) {
  if (causal) {
    return varlen ? launch_nw<D, BF16, true, true>(p, t, stream)
                  : launch_nw<D, BF16, true, false>(p, t, stream);
  }
  return varlen ? launch_nw<D, BF16, false, true>(p, t, stream)
                : launch_nw<D, BF16, false, false>(p, t, stream);
}

hipError_t launch_fwd(const FwdParams& p, int D, bool bf16, bool causal, bool varlen,
                      const FwdTuning& tuning, hipStream_t stream) {
  if (D == 64) {
    return bf16 ? launch_d<64, true>(p, tuning, causal, varlen, stream)
                : launch_d<64, false>(p, tuning, causal, varlen, stream);
  }
  return bf16 ? launch_d<128, true>(p, tuning, causal, varlen, stream)
              : launch_d<128, false>(p, tuning, causal, varlen, stream);
}

}  // namespace sdpa08
