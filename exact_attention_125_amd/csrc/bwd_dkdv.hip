// dK and dV for gfx950 by recomputation: key-owned workgroups, one wave per SIMD.
//
// A workgroup of 4 waves owns KWG keys of one (batch, head); each wave owns KW = 32 KB of
// them (KB = 2 blocks of 32 keys at head dim 64, 1 at 128).  The queries that can see those
// keys stream through LDS in steps of 32.  Per step s and wave:
//
//   S_s  = Q_s K^T + m_s       C[query][key] layout: A = Q_s rows from LDS, B = K^T, and
//                              the per-query m = -LSE / sigma as the initial accumulator
//   dP_s = dO_s V^T - delta_s  A = dO_s rows from LDS, B = V^T, -delta initial accumulator
//   P_s  = 2^(c S_s)           c = sigma log2(e); masked on edge steps (VALU)
//   dS_s = P_s dP_s            (VALU)
//   dV^T += dO_s^T P_s         A = dO_s^T by transposing LDS reads, B = P_s taken from the S
//                              accumulator registers
//   dK^T += Q_s^T dS_s         A = Q_s^T by transposing LDS reads, B = dS_s
//
// Every A operand read from LDS feeds KB MFMAs, one per key block, which keeps LDS issue
// below one instruction per MFMA.  K^T, V^T and the dK^T, dV^T accumulators live in the
// accumulation registers (AGPRs) for the whole kernel, touched only by MFMAs; the VGPRs hold
// the per-step working set.  The step is software-pipelined in two phases, each pairing MFMA
// work with independent VALU work:
//
//   phase 1   dV_s, then S_{s+1}   (MFMA)  with  dS_s     (VALU)
//   phase 2   dK_s, then dP_{s+1}  (MFMA)  with  P_{s+1}  (VALU)
//
// so that the MFMA results the next phase's VALU reads come last in their phase.  Each phase
// also issues, one per MFMA, the LDS reads of the next phase's operands.  Q and dO tiles and
// the per-query statistics arrive by direct global->LDS copies into a ring of kNS stages, kPD
// steps ahead, published by one workgroup barrier per step.  Step s reads tiles s, s+1 and
// s+2 and writes tile s+kPD into the stage of tile s+kPD-kNS (read last in an earlier step);
// the copies of tile s+3 must have landed, in every wave, before the barrier that ends step
// s.  kNS is a power of two, so that the stage of a tile is a mask of its index.
//
// The MFMAs are issued as inline assembly (cdna4.h), so the register dependencies the
// compiler would resolve for the builtins are kept apart by the order written here: VALU
// reads an MFMA result only in the phase after the one that produced it, the products those
// reads need come first in their phase, and the statistics registers an MFMA reads as its
// initial accumulator stay untouched until the phase ends.
//
// The gradients are the derivative of softmax(scale Q K^T + mask) V recomputed tile by
// tile from the saved logsumexp, the recomputation of "PyTorch-CUDA-v2.9镜像中使用
// FlashAttention提升训练速度" ("3. 重计算策略（Recomputation）") and of "告别OOM和训练慢：用Flash
// Attention加速你的PyTorch大模型（含A100环境配置）" §2.2 (only the normalisation statistics are
// kept): dV = P^T dO, dS = P (dO V^T - delta), dK = scale dS^T Q.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "block_list.h"
#include "cdna4.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;   // 4 waves, one per SIMD
constexpr int kBQ = 32;         // queries per step
constexpr int kPD = 5;          // query tiles copied ahead
constexpr int kNS = 8;          // LDS ring stages
static_assert((kNS & (kNS - 1)) == 0 && kNS >= kPD + 1, "a power of two, above kPD");

struct DkdvArgs {
  const char* q;
  const char* k;
  const char* v;
  const char* dout;
  const float* stats;    // m = -LSE / sigma and -rowsum(dO * O) in 32-query blocks (stat_index)
  char* dk;
  char* dv;
  const int* seqlens;    // per-batch lengths (device, may be null: every sequence has n rows)
  const int* cu;         // packed batch: per-batch start rows [B + 1] (device), or null
  int total;             // packed batch: rows per head
  int n;                 // query rows per (batch, head) in memory
  int nk;                // key rows per (batch, head) (n for self-attention, padded batches)
  int heads;
  int n_bh;
  int n_tiles;           // key tiles of KWG keys per head
  int n_units;           // workgroups per head: n_tiles, or ceil(n_tiles / 2) when paired
  int paired;            // a workgroup takes key tiles t and n_tiles - 1 - t
  float c;               // sigma * log2(e)
  float scale;
  int causal, wl, wr;
  int dlo, dhi;          // key j visible to query i iff dlo <= i - j <= dhi (within the sequence)
  const float* slopes;   // ALiBi slopes [heads] (device), read by the ALIBI instances only
  const unsigned char* blocks;   // BLK: block-sparse mask [heads][n_qb][n_kb] of 64 x 64 blocks
  int n_qb, n_kb;
  const unsigned char* kpm;      // KPM: key padding mask [batch][nk] (nonzero = padding key)
};

template <int D>
struct DShape {
  static constexpr int KB = D == 64 ? 2 : 1;       // 32-key blocks per wave
  static constexpr int KW = 32 * KB;               // keys per wave
  static constexpr int KWG = 4 * KW;               // keys per workgroup
  static constexpr int KS = D / 16;                // k-steps over the head dim
  static constexpr int DB = D / 32;                // 32-dim blocks of dK^T, dV^T
  static constexpr int RB = D * 2;                 // bytes per row
  static constexpr int QTILE = kBQ * RB;           // bytes of a Q or dO tile
  static constexpr int STAGE = 2 * QTILE + 1024;   // Q tile, dO tile, statistics (see copy_stats)
  static constexpr int CPT = QTILE / (16 * kThreads);   // 16-byte chunks per thread per tile
  static_assert(QTILE % (16 * kThreads) == 0, "tiles split evenly over the threads");
};

__device__ __forceinline__ f32x16 join4(const f32x4 (&v)[4]) {
  const f32x8 lo = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
  const f32x8 hi = __builtin_shufflevector(v[2], v[3], 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
}

// f(c) for c = B .. E-1, unrolled at compile time (c selects registers)
template <int B, int E, typename F>
__device__ __forceinline__ void slices(F&& f) {
  if constexpr (B < E) {
    f(B);
    slices<B + 1, E>(f);
  }
}

// dK, dV of key tile kt of head bh (the whole workgroup).
// ALIBI (no padded batch; a band with no pair past the diagonal, dlo >= nr - nk, as under a
// causal mask): P carries the forward's ALiBi penalty -slope log2(e) (p - j), p = i + nk - nr the
// query's position, linear in the query index: 2^(c S + La - b2 R), R = 8 (r / 4) + r % 4 of
// accumulator row r, La = -b2 (q0 + 4 hi + nk - nr - j) per key block and step.
// BLK: a block-sparse mask.  The workgroup's 64-key blocks (KWG / 64 of them) select query
// steps; it visits only the steps one of them selects (a list in LDS at `list`, block_list.h),
// and a wave whose block does not select a visited step sees all of its pairs hidden.
// KPM: a key padding mask.  A padding key's column of P and dS is computed like any other and
// touches only its own dK and dV rows, which are written as zeros; a workgroup whose keys are
// all padding writes its zeros without computing.
template <int D, bool BF16, bool PADDED, bool ALIBI = false, bool BLK = false, bool KPM = false>
__device__ __forceinline__ void dkdv_tile(const DkdvArgs& a, char FA_LDS* ring, int FA_LDS* list,
                                          int bh, int kt) {
  static_assert(!(ALIBI && BLK), "no instance takes both");
  static_assert(!(KPM && (ALIBI || BLK || PADDED)), "key padding alone");
  using S = DShape<D>;
  constexpr int KB = S::KB, KS = S::KS, DB = S::DB, RB = S::RB, QTILE = S::QTILE;
  constexpr int STAGE = S::STAGE, CPT = S::CPT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // rows of the head in memory (nr) and of its sequence (n): rows n .. nr-1 are padding, read
  // as zeros through the buffer resources, with zero gradients
  const int nr = a.n;
  // a packed batch: sequence b is rows cu[b] .. cu[b+1]-1 of each head's `total` rows (offsets
  // clamped to [0, total], at most nr rows), with no padding rows to write
  int n = nr, nw = nr;   // sequence rows, rows written
  long head = (long)bh * nr * RB;                              // Q, dO (and K, V, dK, dV)
  if constexpr (PADDED) {
    const int b = bh / a.heads, h = bh - b * a.heads;
    if (a.cu != nullptr) {
      const int c0 = min(max(a.cu[b], 0), a.total);
      const int c1 = min(max(a.cu[b + 1], c0), a.total);
      n = nw = min(c1 - c0, nr);
      head = ((long)h * a.total + c0) * RB;
    } else {
      n = min(max(a.seqlens[b], 0), nr);
    }
  }
  // keys: as many as queries in a padded batch, else nk rows (query i at key position
  // i + nk - n, which the band dlo .. dhi already accounts for)
  const int nkr = PADDED ? n : a.nk;
  const long khead = PADDED ? head : (long)bh * a.nk * RB;     // K, V, dK, dV
  const int head_bytes = n * RB;                               // Q, dO bytes
  const auto rq = make_rsrc(a.q + head, head_bytes);
  const auto rk = make_rsrc(a.k + khead, nkr * RB);
  const auto rv = make_rsrc(a.v + khead, nkr * RB);
  const auto rg = make_rsrc(a.dout + head, head_bytes);
  const int stat_bytes = stat_blocks(nr) * 2 * kStatRows * 4;
  const auto rs = make_rsrc(a.stats + (long)bh * stat_blocks(nr) * 2 * kStatRows, stat_bytes);
  const float c_scale = a.c;
  const float b2 = ALIBI ? a.slopes[bh % a.heads] * kLog2e : 0.f;   // ALiBi slope, base 2

  // ---- this wave's keys: K^T and V^T as B operands (lane: key kw0 + 32 kb + l32, dims of
  // chunk 2 ks + hi), zero beyond the sequence
  const int k_first = kt * S::KWG;
  const int kw0 = k_first + S::KW * wave;
  // ALIBI: la[kb] for query step t (first query 32 (s_begin + t)), set before its P
  float la[KB];
  auto alibi_step = [&](int q0) __attribute__((always_inline)) {
    if constexpr (ALIBI) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        la[kb] = -b2 * (float)(q0 + 4 * hi + a.nk - nr - (kw0 + 32 * kb + l32));
    }
  };
  // KPM: this lane's keys that are padding (or past the sequence); the workgroup skips its
  // work when every one of its keys is
  bool kpad[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) kpad[kb] = false;
  if constexpr (KPM) {
    const unsigned char* kp = a.kpm + (long)(bh / a.heads) * nkr;
    bool all = true;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key = kw0 + 32 * kb + l32;
      kpad[kb] = key >= nkr || kp[key] != 0;
      all = all && kpad[kb];
    }
    int FA_LDS* flags = (int FA_LDS*)list;
    const bool wave_all = __all(all);   // (a vote of every lane: outside the one-lane store)
    if (lane == 0) flags[wave] = wave_all ? 1 : 0;
    wait_lgkmcnt0();   // (the barrier does not wait for LDS writes)
    wg_barrier();
    const bool skip = flags[0] && flags[1] && flags[2] && flags[3];
    wg_barrier();   // every wave has read the flags before a later tile writes them
    if (skip) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int key = kw0 + 32 * kb + l32;
        if (key < nkr) {
          char* dkrow = a.dk + khead + (long)key * RB;
          char* dvrow = a.dv + khead + (long)key * RB;
#pragma unroll
          for (int c16 = 0; c16 < RB / 32; ++c16) {
            *reinterpret_cast<u32x4*>(dkrow + 32 * c16 + 16 * hi) = u32x4{};
            *reinterpret_cast<u32x4*>(dvrow + 32 * c16 + 16 * hi) = u32x4{};
          }
        }
      }
      return;
    }
  }
  i16x8 kreg[KB][KS], vreg[KB][KS];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = (kw0 + 32 * kb + l32) * RB + (2 * ks + hi) * 16;
      kreg[kb][ks] = __builtin_bit_cast(i16x8, buffer_load16(rk, off));
      vreg[kb][ks] = __builtin_bit_cast(i16x8, buffer_load16(rv, off));
    }
  f32x16 dk[KB][DB], dv[KB][DB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dk[kb][db] = f32x16{};
      dv[kb][db] = f32x16{};
    }

  // ---- query steps that can see the workgroup's keys
  // (queries i with dlo <= i - j <= dhi for some key j of the workgroup, within [0, n))
  const int k_last = min(k_first + S::KWG, nkr) - 1;
  const int q_lo = max(0, k_first + a.dlo);
  const int q_hi = min(n, k_last + a.dhi + 1);
  const int s_begin = q_lo / kBQ;
  const int NSTEP = (!PADDED || k_first < n) && q_hi > q_lo ? (q_hi + kBQ - 1) / kBQ - s_begin : 0;
  // BLK: the visited steps, TS of them (entry k: step rel(k) after s_begin and its selections);
  // the entries of steps s + 1 .. s + kPD - 1 are carried in scalars (h1 .. h4), those of later
  // steps read from a window of 64 entries held one per lane
  constexpr int NBW = S::KWG / 64;   // 64-key blocks of the workgroup
  static_assert(S::KWG % 64 == 0, "whole key blocks per workgroup");
  const int own = (S::KW * wave) >> 6;   // this wave's block among them
  int TS = NSTEP;
  int win = 0, h0 = 0, h1 = 1, h2 = 2, h3 = 3, h4 = 4;
  if constexpr (BLK) {
    if (NSTEP > 0)
      TS = build_block_list<NBW, kBQ, kPD, 4>(list, a.blocks + (long)(bh % a.heads) * a.n_qb * a.n_kb, 1,
                                              a.n_kb, k_first >> 6, a.n_kb, s_begin, NSTEP, lane, wave);
    else   // (the prologue's copies read the sentinels)
      TS = build_block_list<NBW, kBQ, kPD, 4>(list, a.blocks, 0, 0, 0, 0, 0, 0, lane, wave);
    win = list[lane];
    h0 = __builtin_amdgcn_readlane(win, 0);
    h1 = __builtin_amdgcn_readlane(win, 1);
    h2 = __builtin_amdgcn_readlane(win, 2);
    h3 = __builtin_amdgcn_readlane(win, 3);
    h4 = __builtin_amdgcn_readlane(win, 4);
  }
  auto rel = [&](int e) __attribute__((always_inline)) { return BLK ? entry_step(e) : e; };

  // ---- per-lane constants
  const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
  const int tr_row = (tg >> 1) * 4 + tr;
  const int tr_byte = (tq & 1) * 8;
  // LDS addresses of this lane's reads, kept per ring stage and moved on by one stage per
  // phase of step s (tile, statistics and 16-row offsets are immediates):
  //   row_a[ks]   A operand rows of a tile (query l32, chunk 2 ks + hi): tile s+1 in phase 1,
  //               tile s+2 in phase 2
  //   st_a        the 16 statistics of this lane's accumulator rows, likewise
  //   tr_a[h][db] transposed halves (rows tr_row + 8 h, dim block db): tile s in phase 1,
  //               tile s+1 in phase 2
  const unsigned ring_a = lds_addr(ring);
  unsigned row_a[KS], st_a, tr_a[2][DB];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) row_a[ks] = ring_a + tile_offset<D>(l32, 2 * ks + hi);
  st_a = ring_a + 2 * QTILE + 64 * hi;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      tr_a[h][db] = ring_a + tile_offset<D>(tr_row + 8 * h, 4 * db + 2 * (tg & 1) + (tq >> 1)) + tr_byte;
  // byte distance from the stage of tile t to that of tile t+1
  auto stage_step = [&](int t) __attribute__((always_inline)) {
    return (t & (kNS - 1)) == kNS - 1 ? -(kNS - 1) * STAGE : STAGE;
  };
  auto advance_rows = [&](int t) __attribute__((always_inline)) {   // stage of t -> of t+1
    const int dlt = stage_step(t);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) row_a[ks] += dlt;
    st_a += dlt;
  };
  auto advance_tr = [&](int t) __attribute__((always_inline)) {
    const int dlt = stage_step(t);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < DB; ++db) tr_a[h][db] += dlt;
  };
  int cp_src[CPT];              // global offset inside a tile of this thread's chunks
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int p = 16 * (tid + kThreads * i);
    const int r = p / RB;
    cp_src[i] = r * RB + ((((p % RB) / 16) ^ chunk_swizzle<D>(r))) * 16;
  }
  // statistics of a 32-query tile, one 256-byte block (m, then -delta): lane L < 16 of every
  // wave copies 16 bytes to LDS slot L (m for L < 8, -delta for 8 <= L < 16; the four waves
  // write the same bytes, which spares a branch and keeps every wave's copy count equal): the
  // values of queries
  // 4 sig(L % 8) .. +3 with sig(j) = 2j (j < 4) or 2(j-4)+1, so that lanes of half hi find the
  // 16 values of their accumulator rows 8 g + 4 hi + 0..3 (g = 0..3) contiguous at slot 4 hi
  // (of the m or -delta half).  Lanes 16..63 read past the buffer and write zeros to slots
  // 16..63, which keeps the copy one full-wave instruction.
  const int jl = lane & 7;
  const int st_src = lane < 16 ? 128 * (lane >> 3) + 16 * (jl < 4 ? 2 * jl : 2 * (jl - 4) + 1)
                               : stat_bytes;

  // ---- copies of pipeline step t (the query tile of entry e, BLK; else tile t) into stage
  // t mod kNS: Q and dO (every wave its share), and the statistics block; past the last tile
  // they read beyond the buffers (zero fills, no traffic) so every step issues the same copies
  auto copy_tiles = [&](int t, int e) __attribute__((always_inline)) {
    const int qt = rel(e);
    const int off = qt < NSTEP ? (s_begin + qt) * kBQ * RB : head_bytes;
    char FA_LDS* st = ring + (t & (kNS - 1)) * STAGE;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      buffer_load16_lds(rq, st + 4096 * i + 1024 * wave, cp_src[i] + off);
      buffer_load16_lds(rg, st + QTILE + 4096 * i + 1024 * wave, cp_src[i] + off);
    }
  };
  auto copy_stats = [&](int t, int e) __attribute__((always_inline)) {
    const int qt = rel(e);
    const int off = qt < NSTEP ? (s_begin + qt) * 2 * kStatRows * 4 : stat_bytes;
    buffer_load16_lds(rs, ring + (t & (kNS - 1)) * STAGE + 2 * QTILE, st_src + off);
  };
  auto issue_copies = [&](int t, int e) __attribute__((always_inline)) {
    copy_stats(t, e);
    copy_tiles(t, e);
  };
  // this wave's copies of tiles up to s+3 have landed (loads complete in order), leaving
  // those of tiles s+4 .. s+kPD in flight (2 CPT tile chunks and one statistics copy each)
  static_assert(kPD >= 3, "the ring holds the three tiles a step reads");
  auto wait_copies = [&]() __attribute__((always_inline)) {
    wait_vmcnt<(kPD - 3) * (2 * CPT + 1)>();
  };

  // ---- operand registers.  All LDS reads in the steps are issued as inline assembly the
  // compiler does not track (it would otherwise wait for every copy in flight into the ring
  // before each read); the waits are explicit fences, counted in LDS reads.  The values look
  // available to the compiler at once, so every piece stays in the register it was read into
  // and is joined with others only where an MFMA uses it, behind the fence.
  i16x8 qa[KS], ga[KS];             // Q, dO rows of a tile (A operands of S, dP)
  // Q^T, dO^T of a tile (A operands of dK, dV) per 16 queries, as the two 4-element halves
  // the transposing reads return
  i16x4 qt_lo[2][DB], qt_hi[2][DB], gt_lo[2][DB], gt_hi[2][DB];
  f32x4 mv[4], ndv[4];              // m and -delta of accumulator rows (initial S, dP)
  f32x16 sacc[KB], dpacc[KB], pv[KB];
  unsigned pk[KB][8], dsk[KB][8];
  constexpr int kTrReads = 2 * 2 * DB;      // transposing reads of one tile
  constexpr int NR = kTrReads + KS + 4;     // LDS reads a phase issues for the next
  static_assert(KS + 4 <= 15 && NR / 2 <= 15, "counted waits fit lgkmcnt");

  // rows (Q at TOFF 0, dO at QTILE) and statistics group WHICH (m, -delta) of the tile
  // row_a / st_a point at (the prologue's reads)
  auto read_rows = [&](auto toff, auto which, i16x8 (&rows)[KS], f32x4 (&stv)[4])
                       __attribute__((always_inline)) {
    constexpr int TOFF = decltype(toff)::value, WHICH = decltype(which)::value;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      rows[ks] = __builtin_bit_cast(i16x8, lds_read16_nowait<TOFF>(row_a[ks]));
    static_for<4>([&](auto gc) __attribute__((always_inline)) {
      constexpr int g = decltype(gc)::value;
      stv[g] = __builtin_bit_cast(f32x4, lds_read16_nowait<128 * WHICH + 16 * g>(st_a));
    });
  };
  // read r of a phase's list: r < kTrReads a transposed half of the tile tr_a points at (at
  // TROFF), then KS rows and 4 statistics vectors of the tile row_a / st_a point at (rows at
  // ROFF, statistics group WHICH)
  auto read_one = [&](auto rc, auto troff, auto roff, auto which, i16x4 (&dlo)[2][DB],
                      i16x4 (&dhi)[2][DB], i16x8 (&rows)[KS], f32x4 (&stv)[4])
                      __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value, TROFF = decltype(troff)::value;
    constexpr int ROFF = decltype(roff)::value, WHICH = decltype(which)::value;
    if constexpr (r < kTrReads) {
      constexpr int kk = r / (2 * DB), db = (r / 2) % DB;
      if constexpr (r % 2 == 0) dlo[kk][db] = lds_read_tr_nowait<TROFF + kk * 16 * RB>(tr_a[0][db]);
      else dhi[kk][db] = lds_read_tr_nowait<TROFF + kk * 16 * RB>(tr_a[1][db]);
    } else if constexpr (r < kTrReads + KS) {
      rows[r - kTrReads] = __builtin_bit_cast(i16x8, lds_read16_nowait<ROFF>(row_a[r - kTrReads]));
    } else {
      constexpr int g = r - kTrReads - KS;
      stv[g] = __builtin_bit_cast(f32x4, lds_read16_nowait<128 * WHICH + 16 * g>(st_a));
    }
  };
  auto read_tr = [&](auto toff, i16x4 (&dlo)[2][DB], i16x4 (&dhi)[2][DB])
                     __attribute__((always_inline)) {
    constexpr int TOFF = decltype(toff)::value;
    static_for<2>([&](auto kkc) __attribute__((always_inline)) {
      constexpr int kk = decltype(kkc)::value;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dlo[kk][db] = lds_read_tr_nowait<TOFF + kk * 16 * RB>(tr_a[0][db]);
        dhi[kk][db] = lds_read_tr_nowait<TOFF + kk * 16 * RB>(tr_a[1][db]);
      }
    });
  };
  using Z = std::integral_constant<int, 0>;
  using O = std::integral_constant<int, 1>;
  using QT = std::integral_constant<int, QTILE>;

  // ---- the four products, one MFMA at a time (m indexes the MFMAs of one product)
  constexpr int NM = KS * KB;       // MFMAs of S or dP
  constexpr int NG = 2 * DB * KB;   // MFMAs of dV or dK
  static_assert(NM == 8 && NG == 8, "phases interleave 16 MFMAs");
  auto mfma_s = [&](auto mc) __attribute__((always_inline)) {        // S = Q K^T + m
    constexpr int m = decltype(mc)::value, ks = m / KB, kb = m % KB;
    if constexpr (ks == 0) mfma_bagpr_init<BF16>(sacc[kb], qa[ks], kreg[kb][ks], join4(mv));
    else mfma_bagpr_acc<BF16>(sacc[kb], qa[ks], kreg[kb][ks]);
  };
  auto mfma_dp = [&](auto mc) __attribute__((always_inline)) {       // dP = dO V^T - delta
    constexpr int m = decltype(mc)::value, ks = m / KB, kb = m % KB;
    if constexpr (ks == 0) mfma_bagpr_init<BF16>(dpacc[kb], ga[ks], vreg[kb][ks], join4(ndv));
    else mfma_bagpr_acc<BF16>(dpacc[kb], ga[ks], vreg[kb][ks]);
  };
  auto mfma_dv = [&](auto mc) __attribute__((always_inline)) {       // dV^T += dO^T P
    constexpr int m = decltype(mc)::value, kk = m / (DB * KB), db = (m / KB) % DB, kb = m % KB;
    const u32x4 b = {pk[kb][4 * kk], pk[kb][4 * kk + 1], pk[kb][4 * kk + 2], pk[kb][4 * kk + 3]};
    const i16x8 op = __builtin_shufflevector(gt_lo[kk][db], gt_hi[kk][db], 0, 1, 2, 3, 4, 5, 6, 7);
    mfma_agpr_acc<BF16>(dv[kb][db], op, __builtin_bit_cast(i16x8, b));
  };
  auto mfma_dk = [&](auto mc) __attribute__((always_inline)) {       // dK^T += Q^T dS
    constexpr int m = decltype(mc)::value, kk = m / (DB * KB), db = (m / KB) % DB, kb = m % KB;
    const u32x4 b = {dsk[kb][4 * kk], dsk[kb][4 * kk + 1], dsk[kb][4 * kk + 2], dsk[kb][4 * kk + 3]};
    const i16x8 op = __builtin_shufflevector(qt_lo[kk][db], qt_hi[kk][db], 0, 1, 2, 3, 4, 5, 6, 7);
    mfma_agpr_acc<BF16>(dk[kb][db], op, __builtin_bit_cast(i16x8, b));
  };

  // ---- the VALU work in slices of two accumulator elements (c = 8 kb + g: elements 2g, 2g+1)
  constexpr int NSL = 8 * KB;
  // P = 2^(c S) for query 8 (i/4) + 4 hi + i%4 of the step
  auto p_slice = [&](int c) __attribute__((always_inline)) {
    const int kb = c >> 3, g = c & 7;
    if constexpr (ALIBI) {
      const float r0 = (float)(8 * ((2 * g) >> 2) + ((2 * g) & 3));
      pv[kb][2 * g] = exp2_fast(__builtin_fmaf(sacc[kb][2 * g], c_scale, __builtin_fmaf(-b2, r0, la[kb])));
      pv[kb][2 * g + 1] =
          exp2_fast(__builtin_fmaf(sacc[kb][2 * g + 1], c_scale, __builtin_fmaf(-b2, r0 + 1.f, la[kb])));
    } else {
      pv[kb][2 * g] = exp2_fast(sacc[kb][2 * g] * c_scale);
      pv[kb][2 * g + 1] = exp2_fast(sacc[kb][2 * g + 1] * c_scale);
    }
    pk[kb][g] = pack2<BF16>(pv[kb][2 * g], pv[kb][2 * g + 1]);
  };
  // On steps that hold hidden pairs, zero them afterwards: a branch around VALU work only, so
  // every step issues the same MFMAs.  Hidden entries were evaluated from scores the mask
  // discards and may be infinite; they are replaced, not scaled.  Rows past the sequence need
  // no mask: their dO and -delta are zero fills, so they add nothing to dV and their dS is 0;
  // keys past the sequence are not stored.  So only the band dlo <= q - key <= dhi is tested:
  // q - key - dlo = u + 8 (i/4) + i%4 with u per lane, compared unsigned against dhi - dlo.
  //
  // Where only a lower band edge on a multiple of 32 crosses the step (the causal diagonal, a
  // right window of a multiple of 32), every 32x32 block of the step is wholly visible,
  // wholly hidden or cut along its diagonal: q - key = x - 32 kb + (row - column) with x =
  // q0 - kw0 a multiple of 32 and row - column in [-31, 31].  Those blocks take constant lane
  // masks instead of compares.
  // (hide: every pair of the step hidden)
  auto mask_step = [&](int t, bool hide) __attribute__((always_inline)) {
    keep_branch();   // not worth running on every step
    const int q0 = (s_begin + t) * kBQ;
    const int x = q0 - kw0;   // wave-uniform
    if (hide || ((a.dlo & 31) == 0 && a.dhi - x >= 31)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int lo = hide ? 32 : a.dlo - x + 32 * kb;   // visible iff row - column >= lo
        if (lo >= 32) {
#pragma unroll
          for (int i = 0; i < 16; ++i) pv[kb][i] = 0.f;
#pragma unroll
          for (int g = 0; g < 8; ++g) pk[kb][g] = 0u;
        } else if (lo == 0) {
          static_for<16>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            pv[kb][i] = keep_lanes(pv[kb][i], diag_lanes<false>(i));
          });
#pragma unroll
          for (int g = 0; g < 8; ++g) pk[kb][g] = pack2<BF16>(pv[kb][2 * g], pv[kb][2 * g + 1]);
        }
      }
      return;
    }
    const unsigned span = (unsigned)(a.dhi - a.dlo);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int u = q0 + 4 * hi - (kw0 + 32 * kb + l32) - a.dlo;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pv[kb][i] = (unsigned)(u + 8 * (i >> 2) + (i & 3)) <= span ? pv[kb][i] : 0.f;
#pragma unroll
      for (int g = 0; g < 8; ++g) pk[kb][g] = pack2<BF16>(pv[kb][2 * g], pv[kb][2 * g + 1]);
    }
  };
  // dS = P (dP - delta)
  auto ds_slice = [&](int c) __attribute__((always_inline)) {
    const int kb = c >> 3, g = c & 7;
    dsk[kb][g] = pack2<BF16>(pv[kb][2 * g] * dpacc[kb][2 * g], pv[kb][2 * g + 1] * dpacc[kb][2 * g + 1]);
  };
  // Some pair of step t lies outside the band unless t_in_lo <= t <= t_in_hi: the step's
  // queries q0 .. q0+31 (q0 = 32 (s_begin + t)) against this wave's keys need
  // q0 - (kw0 + KW - 1) >= dlo and q0 + 31 - kw0 <= dhi, solved for t once (the shifts are
  // floor divisions, also below zero), so each step tests two scalars.
  static_assert(kBQ == 32, "steps of 32 queries");
  const int t_in_lo = ((a.dlo + kw0 + S::KW - 1 + 31) >> 5) - s_begin;
  const int t_in_hi = ((a.dhi + kw0 - 31) >> 5) - s_begin;
  auto edge_step = [&](int t) __attribute__((always_inline)) {
    return t < t_in_lo || t > t_in_hi;
  };

  // ---- phases: each MFMA followed by its share of the phase's VALU slices, with a
  // scheduling fence after each pair so that the issue order is the written one
  auto pin_phase1 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int g = 0; g < 8; ++g) pin(dsk[kb][g]);
#pragma unroll
    for (int g = 0; g < 4; ++g) keep(mv[g]);   // read by this phase's products: kept until here
  };
  auto pin_phase2 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      pin(pv[kb]);
#pragma unroll
      for (int g = 0; g < 8; ++g) pin(pk[kb][g]);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) keep(ndv[g]);
  };
  // Every step computes S, dP and P of the following tile; after the last step that tile is
  // the zero fill past the sequence and its values go unused.  One MFMA sequence per phase,
  // with no branch around any of it, keeps each accumulator in one set of registers.
  //
  // Counted waits: a phase starts when the transposed halves the previous phase read have
  // landed (its KS + 4 rows and statistics reads may still be in flight) and runs its second
  // product once those have landed too (its own first NR / 2 reads may still be in flight).
  //
  // phase 1 of step s: dV_s, S_{s+1} | dS_s; reads Q_s^T, dO_{s+1} rows, -delta_{s+1}; copies
  // of tile s + kPD
  // (ek: the entry of step s + kPD, whose tiles it copies)
  auto phase1 = [&](int s, int ek) __attribute__((always_inline)) {
    wait_lgkmcnt_fence<KS + 4>();
    static_for<NG + NM>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m == NG) wait_lgkmcnt_fence<NR / 2>();   // Q_{s+1} rows and m have landed
      if constexpr (m < NG) mfma_dv(std::integral_constant<int, m>{});
      else mfma_s(std::integral_constant<int, m - NG>{});
      slices<m * NSL / (NG + NM), (m + 1) * NSL / (NG + NM)>(ds_slice);
      static_for<(m + 1) * NR / (NG + NM) - m * NR / (NG + NM)>([&](auto jc) __attribute__((always_inline)) {
        read_one(std::integral_constant<int, m * NR / (NG + NM) + decltype(jc)::value>{}, Z{}, QT{}, O{},
                 qt_lo, qt_hi, ga, ndv);
      });
      if constexpr (m == 1) copy_tiles(s + kPD, ek);
      __builtin_amdgcn_sched_barrier(0);
    });
    pin_phase1();
  };
  // phase 2 of step s: dK_s, dP_{s+1} | P_{s+1}; reads dO_{s+1}^T, Q_{s+2} rows, m_{s+2}.  The
  // slices start after the second MFMA: S_{s+1} was the last product of phase 1.
  auto phase2 = [&]() __attribute__((always_inline)) {
    wait_lgkmcnt_fence<KS + 4>();
    static_for<NG + NM>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m == NG) wait_lgkmcnt_fence<NR / 2>();   // dO_{s+1} rows and -delta have landed
      if constexpr (m < NG) mfma_dk(std::integral_constant<int, m>{});
      else mfma_dp(std::integral_constant<int, m - NG>{});
      constexpr int W = NG + NM - 2;
      if constexpr (m >= 2) slices<(m - 2) * NSL / W, (m - 1) * NSL / W>(p_slice);
      static_for<(m + 1) * NR / (NG + NM) - m * NR / (NG + NM)>([&](auto jc) __attribute__((always_inline)) {
        read_one(std::integral_constant<int, m * NR / (NG + NM) + decltype(jc)::value>{}, QT{}, Z{}, Z{},
                 gt_lo, gt_hi, qa, mv);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    pin_phase2();
  };

  // ---- prologue: tiles 0..kPD-1, then S_0, dP_0, P_0 and the operands of step 0's phase 1
  static_assert(kPD == 5, "entries of steps 0 .. 4 in h0 .. h4");
  issue_copies(0, h0);
  issue_copies(1, h1);
  issue_copies(2, h2);
  issue_copies(3, h3);
  issue_copies(4, h4);
  // K^T, V^T and the accumulators into the AGPRs only now, so that waiting for the K and V rows
  // does not hold back the copies; the wait states after separate those writes from the first
  // product
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      in_agpr(kreg[kb][ks]);
      in_agpr(vreg[kb][ks]);
    }
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      in_agpr(dk[kb][db]);
      in_agpr(dv[kb][db]);
    }
  mfma_operand_wait();
  wait_vmcnt<0>();
  wg_barrier();
  if (TS > 0) {
    read_rows(Z{}, Z{}, qa, mv);
    read_rows(QT{}, O{}, ga, ndv);
    wait_lgkmcnt0_fence();
    static_for<NM>([&](auto mc) __attribute__((always_inline)) { mfma_s(mc); });
    static_for<NM>([&](auto mc) __attribute__((always_inline)) { mfma_dp(mc); });
    // the products' results are read by VALU below
    mfma_result_wait();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      pin(sacc[kb]);
      pin(dpacc[kb]);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      keep(mv[g]);
      keep(ndv[g]);
    }
    alibi_step(s_begin * kBQ);
    slices<0, NSL>(p_slice);
    const bool hide = BLK && !entry_selected(h0, own);
    if (hide || edge_step(rel(h0))) mask_step(rel(h0), hide);
    pin_phase2();
  }
  read_tr(QT{}, gt_lo, gt_hi);       // dO_0^T
  advance_rows(0);
  read_rows(Z{}, Z{}, qa, mv);       // Q_1 rows, m_1
  wait_lgkmcnt0_fence();
  // from here: tr_a at tile s, row_a / st_a at tile s+1 when step s begins

  // ---- steps: one barrier each
  for (int s = 0; s < TS; ++s) {
    int ek = s + kPD, e1 = s + 1;
    if constexpr (BLK) {
      if (((s + kPD) & 63) == 0) win = list[s + kPD + lane];   // the next window (rare)
      ek = __builtin_amdgcn_readlane(win, (s + kPD) & 63);
      e1 = h1;
      h1 = h2;
      h2 = h3;
      h3 = h4;
      h4 = ek;
    }
    copy_stats(s + kPD, ek);         // before the phase: its branch stays out of the MFMA sequence
    phase1(s, ek);
    advance_tr(s);                   // tile s   -> s+1
    advance_rows(s + 1);             // tile s+1 -> s+2
    alibi_step((s_begin + s + 1) * kBQ);
    phase2();
    const bool hide = BLK && !entry_selected(e1, own);
    if (s + 1 < TS && (hide || edge_step(rel(e1)))) {
      mask_step(rel(e1), hide);
      pin_phase2();
    }
    wait_copies();
    wg_barrier();
  }
  wait_lgkmcnt0();
  wait_vmcnt<0>();   // no copy may land after the workgroup ends

  // ---- epilogue: lane holds key kw0 + 32 kb + l32, dims 32 db + 8 g + 4 hi + 0..3.  The
  // accumulators were last written by products; keep their reads the required distance away.
  mfma_result_wait();
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      in_agpr(dk[kb][db]);
      in_agpr(dv[kb][db]);
    }
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int key = kw0 + 32 * kb + l32;
    if (key < (PADDED ? nw : nkr)) {
      char* dkrow = a.dk + khead + (long)key * RB;
      char* dvrow = a.dv + khead + (long)key * RB;
      const float sc = a.scale;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dim = 32 * db + 8 * g + 4 * hi;
          u32x2 wk = {pack2<BF16>(dk[kb][db][4 * g + 0] * sc, dk[kb][db][4 * g + 1] * sc),
                      pack2<BF16>(dk[kb][db][4 * g + 2] * sc, dk[kb][db][4 * g + 3] * sc)};
          u32x2 wv = {pack2<BF16>(dv[kb][db][4 * g + 0], dv[kb][db][4 * g + 1]),
                      pack2<BF16>(dv[kb][db][4 * g + 2], dv[kb][db][4 * g + 3])};
          if ((PADDED && key >= n) || (KPM && kpad[kb])) wk = wv = u32x2{};   // padding keys: zero gradients
          *reinterpret_cast<u32x2*>(dkrow + dim * 2) = wk;
          *reinterpret_cast<u32x2*>(dvrow + dim * 2) = wv;
        }
    }
  }
}

// Under a causal mask (no left window) the number of query steps falls linearly with the key
// tile, so tiles t and n_tiles - 1 - t together take the same time for every t: paired, the
// workgroups are of equal length and fill the chip evenly.
// PADDED: a padded batch (per-batch lengths), a separate instance
template <int D, bool BF16, bool PADDED, bool ALIBI = false, bool BLK = false, bool KPM = false>
__global__ __launch_bounds__(kThreads) void dkdv_main_kernel(DkdvArgs a) {
  constexpr int kRing = kNS * DShape<D>::STAGE;
  constexpr int kExtra = BLK ? block_list_bytes<DShape<D>::KWG / 64>() : KPM ? 16 : 0;
  __shared__ __attribute__((aligned(1024))) char lds_raw[kRing + kExtra];
  char FA_LDS* ring = (char FA_LDS*)lds_raw;
  int FA_LDS* list = (int FA_LDS*)(lds_raw + kRing);
  int bh, t;
  xcd_tile_order(blockIdx.x, a.n_bh, a.n_units, bh, t);
  const int n_pass = a.paired && t != a.n_tiles - 1 - t ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
    if (pass > 0) wg_barrier();   // every wave is done with the ring before it is refilled
    dkdv_tile<D, BF16, PADDED, ALIBI, BLK, KPM>(a, ring, list, bh, pass == 0 ? t : a.n_tiles - 1 - t);
  }
}

// nq query rows over nk key rows (dense operands); query i at key position i + nk - nq
template <int D, bool BF16>
hipError_t launch(const BwdParams& p, int nq, int nk, hipStream_t stream) {
  using S = DShape<D>;
  DkdvArgs a;
  a.q = static_cast<const char*>(p.q);
  a.k = static_cast<const char*>(p.k);
  a.v = static_cast<const char*>(p.v);
  a.dout = static_cast<const char*>(p.dout);
  a.stats = p.stats;
  a.dk = static_cast<char*>(p.dk);
  a.dv = static_cast<char*>(p.dv);
  a.seqlens = p.seqlens;
  a.cu = p.cu;
  a.total = p.total;
  a.n = nq;
  a.nk = nk;
  a.heads = p.H;
  a.n_bh = p.B * p.H;
  a.n_tiles = (nk + S::KWG - 1) / S::KWG;
  a.c = (float)((double)softmax_sigma(p.scale) * 1.4426950408889634);
  a.scale = p.scale;
  a.causal = p.causal;
  a.wl = p.window_left;
  a.wr = p.causal ? 0 : p.window_right;
  // a window of kUnbounded or more is no bound: every i - j of a sequence the library takes
  // (N < 2^24) lies inside it, and dhi - dlo stays below 2^32
  constexpr int kUnbounded = 1 << 30;
  const int wr = p.window_right < 0 ? kUnbounded : std::min(p.window_right, kUnbounded);
  const int wl = p.window_left < 0 ? kUnbounded : std::min(p.window_left, kUnbounded);
  // the band in query-index space: positions are indices + nk - nq
  a.dlo = (p.causal ? 0 : -wr) - (nk - nq);
  a.dhi = wl - (nk - nq);
  const int half = (a.n_tiles + 1) / 2;
  a.paired = p.causal && p.window_left < 0 && (long)a.n_bh * half >= 256;
  a.n_units = a.paired ? half : a.n_tiles;
  a.slopes = p.slopes;
  a.blocks = p.blocks;
  a.kpm = p.kpm;
  a.n_qb = (nq + 63) / 64;
  a.n_kb = (nk + 63) / 64;
  const long blocks = (long)a.n_bh * a.n_units;
  if (p.slopes != nullptr)   // (no padded batch takes ALiBi or a block mask)
    hipLaunchKernelGGL((dkdv_main_kernel<D, BF16, false, true>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, a);
  else if (p.blocks != nullptr)
    hipLaunchKernelGGL((dkdv_main_kernel<D, BF16, false, false, true>), dim3((unsigned)blocks),
                       dim3(kThreads), 0, stream, a);
  else if (p.kpm != nullptr)
    hipLaunchKernelGGL((dkdv_main_kernel<D, BF16, false, false, false, true>), dim3((unsigned)blocks),
                       dim3(kThreads), 0, stream, a);
  else if (p.seqlens != nullptr || p.cu != nullptr)
    hipLaunchKernelGGL((dkdv_main_kernel<D, BF16, true>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((dkdv_main_kernel<D, BF16, false>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dkdv_main(const BwdParams& p, hipStream_t stream) {
  return launch_dkdv_main_kv(p, p.N, p.N, stream);
}

hipError_t launch_dkdv_main_kv(const BwdParams& p, int nq, int nk, hipStream_t stream) {
  if (p.D == 64) return p.bf16 ? launch<64, true>(p, nq, nk, stream) : launch<64, false>(p, nq, nk, stream);
  return p.bf16 ? launch<128, true>(p, nq, nk, stream) : launch<128, false>(p, nq, nk, stream);
}

}  // namespace fa
