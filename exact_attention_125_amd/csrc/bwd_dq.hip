// dQ for gfx950 by recomputation: query-owned workgroups of one wave per SIMD.
//
// A workgroup of 4 waves owns QWG queries of one (batch, head); each wave owns QW = 32 of
// them, one query per lane.  At head dim 64 the working set fits in half of a SIMD's registers,
// so two workgroups share a CU and each SIMD issues the VALU work of two waves (a single wave
// issues VALU instructions at half the rate the SIMD can retire them); at 128 one does.
// The keys those queries can see stream through LDS in steps of 32.  Per step s and wave
// (C[key][query] layouts, so a lane's accumulator entries all belong to its query):
//
//   S_s^T  = K_s Q^T             A = K_s rows from LDS, B = Q^T
//   dP_s^T = V_s dO^T - delta    A = V_s rows from LDS, B = dO^T; -delta of the lane's query
//                                as the initial accumulator
//   P_s    = 2^(c S_s + c m)     c = sigma log2(e), m = -LSE / sigma of the lane's query
//   dS_s   = P_s dP_s
//   dQ^T  += K_s^T dS_s^T        A = K_s^T by transposing LDS reads, B = dS_s from the
//                                accumulator registers
//
// Q^T, dO^T and the dQ^T accumulators live in the accumulation registers (AGPRs) for the
// whole kernel, touched only by MFMAs.  The step is software-pipelined in two phases:
//
//   phase 1   dQ_{s-1}, then dP_s   (MFMA)  with  P_s    (VALU)
//   phase 2   S_{s+1}               (MFMA)  with  dS_s   (VALU)
//
// and each phase issues, between its MFMAs, the LDS reads of later operands: phase 1 (in
// its second half, once dQ_{s-1} has taken its operands) the K_{s+1} rows and K_s^T halves,
// phase 2 the V_{s+1} rows.  K and V tiles arrive by direct global->LDS copies into a ring of
// kNS stages, kPD steps ahead, published by one workgroup barrier per step.  Step s reads
// tiles s and s+1 and writes tile s+kPD into the stage of tile s-1.  As in the dK/dV kernel,
// the MFMAs are inline assembly with register dependencies kept apart by the written order,
// and all LDS reads in the steps are untracked with counted waits.
//
// dQ = scale dS K, the query-side derivative of softmax(scale Q K^T + mask) V recomputed from
// the saved logsumexp: the recomputation of "PyTorch-CUDA-v2.9镜像中使用FlashAttention提升训练
// 速度" ("3. 重计算策略（Recomputation）") and of "告别OOM和训练慢：用Flash Attention加速你的
// PyTorch大模型（含A100环境配置）" §2.2.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "block_list.h"
#include "cdna4.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;   // 4 waves, one per SIMD per workgroup
constexpr int kBK = 32;         // keys per step
constexpr int kPD = 4;          // key tiles copied ahead
constexpr int kNS = kPD + 1;    // LDS ring stages

struct DqArgs {
  const char* q;
  const char* k;
  const char* v;
  const char* dout;
  const float* stats;    // m = -LSE / sigma and -rowsum(dO * O) in 32-query blocks (stat_index)
  // or, with stats_out set, the kernel forms those statistics of its own queries from O and
  // LSE and writes them to stats_out for the dK/dV kernel
  float* stats_out;
  const char* o;
  const float* lse;      // [B, H, n] (a packed batch: [H, total])
  float sigma;           // softmax_scale kept away from zero (softmax_sigma)
  char* dq;
  const int* seqlens;    // per-batch lengths (device, may be null: every sequence has n rows)
  const int* cu;         // packed batch: per-batch start rows [B + 1] (device), or null
  int total;             // packed batch: rows per head
  int n;                 // query rows per (batch, head) in memory
  int nk;                // key rows per (batch, head) (n for self-attention, padded batches)
  int off;               // key position of query 0 (nk - n)
  int heads;
  int n_bh;
  int n_tiles;           // query tiles of QWG queries per head
  int n_units;           // workgroups per head: n_tiles, or ceil(n_tiles / 2) when paired
  int paired;            // a workgroup takes query tiles t and n_tiles - 1 - t
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
struct QShape {
  static constexpr int QB = 1;                     // 32-query blocks per wave
  static constexpr int QW = 32 * QB;               // queries per wave
  static constexpr int QWG = 4 * QW;               // queries per workgroup
  static constexpr int KS = D / 16;                // k-steps over the head dim
  static constexpr int DB = D / 32;                // 32-dim blocks of dQ^T
  static constexpr int RB = D * 2;                 // bytes per row
  static constexpr int KTILE = kBK * RB;           // bytes of a K or V tile
  static constexpr int STAGE = 2 * KTILE;          // K tile, V tile
  static constexpr int CPT = KTILE / (16 * kThreads);   // 16-byte chunks per thread per tile
  static_assert(KTILE % (16 * kThreads) == 0, "tiles split evenly over the threads");
};

// f(c) for c = B .. E-1, unrolled at compile time (c selects registers)
template <int B, int E, typename F>
__device__ __forceinline__ void dq_slices(F&& f) {
  if constexpr (B < E) {
    f(B);
    dq_slices<B + 1, E>(f);
  }
}

// dQ of query tile qt of head bh (the whole workgroup).
// ALIBI (no padded batch; a band with no pair past the diagonal, as under a causal mask): P
// carries the forward's ALiBi penalty -slope log2(e) (p - j), p = q + off the query's position,
// linear in the key index: 2^(c S + Lq + b2 R), R = 8 (r / 4) + r % 4 of accumulator row r,
// Lq = c m - b2 (p - k0 - 4 hi) per query block and step (keys k0 ..).
// BLK: a block-sparse mask.  The workgroup's two 64-query blocks select key steps; it visits
// only the steps one of them selects (a list in LDS at `list`, block_list.h), and a wave whose
// block does not select a visited step sees all of its pairs hidden.
// KPM: a key padding mask.  The workgroup gathers one padding word per key step (bit k: key k
// of the step is padding) into LDS at `list`, drops the leading and trailing steps made only of
// padding, and zeroes the probabilities of padding keys in the steps that have some, one
// v_cndmask per element with a scalar lane mask.
template <int D, bool BF16, bool PADDED, bool ALIBI = false, bool BLK = false, bool KPM = false>
__device__ __forceinline__ void dq_tile(const DqArgs& a, char FA_LDS* ring, int FA_LDS* list, int bh,
                                        int qt) {
  static_assert(!(ALIBI && BLK), "no instance takes both");
  static_assert(!(KPM && (ALIBI || BLK || PADDED)), "key padding alone");
  using S = QShape<D>;
  constexpr int QB = S::QB, KS = S::KS, DB = S::DB, RB = S::RB, KTILE = S::KTILE;
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
  long head = (long)bh * nr * RB;                              // Q, dO, O, dQ (and K, V)
  long lse_row = (long)bh * nr;                                // LSE of query 0
  if constexpr (PADDED) {
    const int b = bh / a.heads, h = bh - b * a.heads;
    if (a.cu != nullptr) {
      const int c0 = min(max(a.cu[b], 0), a.total);
      const int c1 = min(max(a.cu[b + 1], c0), a.total);
      n = nw = min(c1 - c0, nr);
      head = ((long)h * a.total + c0) * RB;
      lse_row = (long)h * a.total + c0;
    } else {
      n = min(max(a.seqlens[b], 0), nr);
    }
  }
  // keys: as many as queries in a padded batch, else nk rows, query i at key position i + off
  const int nkr = PADDED ? n : a.nk;
  const int off = PADDED ? 0 : a.off;
  const long khead = PADDED ? head : (long)bh * a.nk * RB;     // K, V
  const int head_bytes = nkr * RB;                             // K, V bytes
  const auto rq = make_rsrc(a.q + head, n * RB);
  const auto rk = make_rsrc(a.k + khead, head_bytes);
  const auto rv = make_rsrc(a.v + khead, head_bytes);
  const auto rg = make_rsrc(a.dout + head, n * RB);
  const Mask mk{nkr, a.causal, a.wl, a.wr};
  const float c_scale = a.c;
  const float b2 = ALIBI ? a.slopes[bh % a.heads] * kLog2e : 0.f;   // ALiBi slope, base 2

  // ---- this wave's queries: Q^T and dO^T as B operands (lane: query qw0 + 32 qb + l32, dims
  // of chunk 2 ks + hi), zero beyond the sequence; their statistics as lane scalars
  const int q_first = qt * S::QWG;
  const int qw0 = q_first + S::QW * wave;
  i16x8 qreg[QB][KS], greg[QB][KS];
  float lse_in[QB], nd_in[QB];   // statistics as loaded (row 0's beyond the sequence)
  // with a.stats_out the kernel forms the statistics of its queries itself: lse_in holds the
  // LSE until then, ov the lane's chunks of the O rows
  const bool form_stats = a.stats_out != nullptr;
  const auto ro = make_rsrc(a.o + head, n * RB);
  const auto rl = make_rsrc(a.lse + lse_row, 4 * n);
  u32x4 ov[QB][KS];
  float stat_out[QB];   // the lane's value of the wave's statistics block: m (lower half) or -delta
  float cm[QB];                  // c m = -log2(e) LSE, set after the prologue copies
  float lq0[QB], lq[QB];         // ALIBI: c m - b2 (p - 4 hi), and Lq of the current step
  f32x16 ndv[QB];                // -delta, the initial accumulator of dP, likewise
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qw0 + 32 * qb + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = q * RB + (2 * ks + hi) * 16;
      qreg[qb][ks] = __builtin_bit_cast(i16x8, buffer_load16(rq, off));
      greg[qb][ks] = __builtin_bit_cast(i16x8, buffer_load16(rg, off));
    }
    if (form_stats) {   // O rows (chunks as dO's) and LSE, used once the copies are issued
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ov[qb][ks] = buffer_load16(ro, q * RB + (2 * ks + hi) * 16);
      lse_in[qb] = buffer_load_f32(rl, 4 * q);   // (zero past the sequence, not used there)
    } else {
      const long r = stat_index(bh, nr, q < n ? q : 0);
      lse_in[qb] = a.stats[r];
      nd_in[qb] = a.stats[r + kStatRows];
    }
  }
  f32x16 dqacc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) dqacc[qb][db] = f32x16{};

  // ---- key steps the workgroup's queries can see
  int k_lo, k_hi;
  mk.key_range(q_first + off, min(q_first + S::QWG, n) - 1 + off, k_lo, k_hi);
  int s_begin = k_lo / kBK;
  int NSTEP = (!PADDED || q_first < n) && k_hi > k_lo ? (k_hi + kBK - 1) / kBK - s_begin : 0;
  // KPM: padding word of step s at pwords[s + pw_off]; the first and past-last steps with a key
  unsigned FA_LDS* pwords = (unsigned FA_LDS*)list;
  int pw_off = 0;
  if constexpr (KPM) {
    int FA_LDS* ptrim = (int FA_LDS*)(pwords + kListMax + 64);
    const unsigned char* kp = a.kpm + (long)(bh / a.heads) * nkr;
    for (int s = wave; s < NSTEP; s += 4) {
      const int j = (s_begin + s) * kBK + l32;
      const bool pad = hi != 0 || j >= nkr || kp[j] != 0;
      const unsigned long long w = __ballot(pad);
      if (lane == 0) pwords[s] = (unsigned)w;
    }
    wait_lgkmcnt0();   // (the barrier does not wait for LDS writes)
    wg_barrier();
    if (wave == 0) {
      int first = NSTEP, last = -1;
      for (int c = 0; c < NSTEP; c += 64) {
        const bool live = c + lane < NSTEP && pwords[c + lane] != 0xffffffffu;
        const unsigned long long b = __ballot(live);
        if (b != 0) {
          if (first == NSTEP) first = c + __builtin_ctzll(b);
          last = c + 63 - __builtin_clzll(b);
        }
      }
      if (lane == 0) {
        ptrim[0] = first;
        ptrim[1] = last + 1;
      }
    }
    wait_lgkmcnt0();
    wg_barrier();
    const int first = __builtin_amdgcn_readfirstlane(ptrim[0]);
    const int past = __builtin_amdgcn_readfirstlane(ptrim[1]);
    s_begin += first;
    NSTEP = past > first ? past - first : 0;
    pw_off = first;
  }
  // BLK: the visited steps, TS of them (entry k: step rel(k) after s_begin and its selections);
  // the entries of steps s .. s + kPD - 1 are carried in scalars (h0 .. h3), those of later
  // steps read from a window of 64 entries held one per lane
  int TS = NSTEP;
  int win = 0, h0 = 0, h1 = 1, h2 = 2, h3 = 3;
  if constexpr (BLK) {
    if (NSTEP > 0)
      TS = build_block_list<2, kBK, kPD, 4>(list, a.blocks + (long)(bh % a.heads) * a.n_qb * a.n_kb,
                                            a.n_kb, 1, q_first >> 6, a.n_qb, s_begin, NSTEP, lane, wave);
    else   // (the prologue's copies read the sentinels)
      TS = build_block_list<2, kBK, kPD, 4>(list, a.blocks, 0, 0, 0, 0, 0, 0, lane, wave);
    win = list[lane];
    h0 = __builtin_amdgcn_readlane(win, 0);
    h1 = __builtin_amdgcn_readlane(win, 1);
    h2 = __builtin_amdgcn_readlane(win, 2);
    h3 = __builtin_amdgcn_readlane(win, 3);
  }
  auto rel = [&](int e) __attribute__((always_inline)) { return BLK ? entry_step(e) : e; };

  // ---- per-lane LDS addresses, moved on by one ring stage per step:
  //   row_a[ks]   A operand rows (key l32, chunk 2 ks + hi) in the stage of tile s+1 (K at
  //               +0, V at +KTILE)
  //   tr_a[h][db] transposed halves (rows tr_row + 8 h, dim block db) in the stage of tile s
  const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
  const int tr_row = (tg >> 1) * 4 + tr;
  const int tr_byte = (tq & 1) * 8;
  const unsigned ring_a = lds_addr(ring);
  unsigned row_a[KS], tr_a[2][DB];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) row_a[ks] = ring_a + tile_offset<D>(l32, 2 * ks + hi);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      tr_a[h][db] = ring_a + tile_offset<D>(tr_row + 8 * h, 4 * db + 2 * (tg & 1) + (tq >> 1)) + tr_byte;
  auto stage_step = [&](int t) __attribute__((always_inline)) {   // stage of t -> of t+1
    return (t % kNS) == kNS - 1 ? -(kNS - 1) * STAGE : STAGE;
  };
  int cp_src[CPT];              // global offset inside a tile of this thread's chunks
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int p = 16 * (tid + kThreads * i);
    const int r = p / RB;
    cp_src[i] = r * RB + ((((p % RB) / 16) ^ chunk_swizzle<D>(r))) * 16;
  }

  // ---- copies of pipeline step t (the key tile of entry e, BLK; else tile t) into stage
  // t % kNS; past the last tile they read beyond the buffers (zero fills, no traffic) so every
  // step issues the same copies
  auto issue_copies = [&](int t, int e) __attribute__((always_inline)) {
    const int kt = rel(e);
    const int off = kt < NSTEP ? (s_begin + kt) * kBK * RB : head_bytes;
    char FA_LDS* st = ring + (t % kNS) * STAGE;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      buffer_load16_lds(rk, st + 4096 * i + 1024 * wave, cp_src[i] + off);
      buffer_load16_lds(rv, st + KTILE + 4096 * i + 1024 * wave, cp_src[i] + off);
    }
  };
  // this wave's copies of tiles up to s+2 have landed, those of s+3 .. s+kPD in flight
  static_assert(kPD >= 2, "the ring holds the two tiles a step reads");
  auto copy_tiles = issue_copies;

  // ---- operand registers (untracked LDS reads; joined with others only at the MFMA)
  i16x8 ka[KS], va[KS];             // K_{s+1}, V_s rows (A operands of S^T, dP^T)
  i16x4 kt_lo[2][DB], kt_hi[2][DB]; // K^T halves of a tile (A operand of dQ^T)
  f32x16 sacc[QB], dpacc[QB], pv[QB];
  unsigned dsk[QB][8];
  constexpr int kTrReads = 2 * 2 * DB;
  constexpr int NR1 = KS + kTrReads;        // reads of phase 1's second half: K rows, K^T
  constexpr int kTrWait = kTrReads < 15 ? kTrReads : 15;
  static_assert(KS <= 15, "counted waits fit lgkmcnt");

  auto read_rows = [&](const unsigned (&addr)[KS], auto toff, i16x8 (&rows)[KS])
                       __attribute__((always_inline)) {
    constexpr int TOFF = decltype(toff)::value;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      rows[ks] = __builtin_bit_cast(i16x8, lds_read16_nowait<TOFF>(addr[ks]));
  };
  // read r of phase 1's list: K_{s+1} rows (r < KS), then the K_s^T halves
  auto read_one = [&](auto rc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    if constexpr (r < KS) {
      ka[r] = __builtin_bit_cast(i16x8, lds_read16_nowait<0>(row_a[r]));
    } else {
      constexpr int t = r - KS, kk = t / (2 * DB), db = (t / 2) % DB;
      if constexpr (t % 2 == 0) kt_lo[kk][db] = lds_read_tr_nowait<kk * 16 * RB>(tr_a[0][db]);
      else kt_hi[kk][db] = lds_read_tr_nowait<kk * 16 * RB>(tr_a[1][db]);
    }
  };
  using Z = std::integral_constant<int, 0>;
  using KT = std::integral_constant<int, KTILE>;

  // ---- the three products, one MFMA at a time
  constexpr int NM = KS * QB;       // MFMAs of S^T or dP^T
  constexpr int NG = 2 * DB * QB;   // MFMAs of dQ^T
  static_assert(NM == NG && NM >= 4, "phases interleave products of equal length");
  auto mfma_s = [&](auto mc) __attribute__((always_inline)) {        // S^T = K Q^T
    constexpr int m = decltype(mc)::value, ks = m / QB, qb = m % QB;
    if constexpr (ks == 0) mfma_bagpr_first<BF16>(sacc[qb], ka[ks], qreg[qb][ks]);
    else mfma_bagpr_acc<BF16>(sacc[qb], ka[ks], qreg[qb][ks]);
  };
  auto mfma_dp = [&](auto mc) __attribute__((always_inline)) {       // dP^T = V dO^T - delta
    constexpr int m = decltype(mc)::value, ks = m / QB, qb = m % QB;
    if constexpr (ks == 0) mfma_bagpr_init<BF16>(dpacc[qb], va[ks], greg[qb][ks], ndv[qb]);
    else mfma_bagpr_acc<BF16>(dpacc[qb], va[ks], greg[qb][ks]);
  };
  auto mfma_dq = [&](auto mc) __attribute__((always_inline)) {       // dQ^T += K^T dS^T
    constexpr int m = decltype(mc)::value, kk = m / (DB * QB), db = (m / QB) % DB, qb = m % QB;
    const u32x4 b = {dsk[qb][4 * kk], dsk[qb][4 * kk + 1], dsk[qb][4 * kk + 2], dsk[qb][4 * kk + 3]};
    const i16x8 op = __builtin_shufflevector(kt_lo[kk][db], kt_hi[kk][db], 0, 1, 2, 3, 4, 5, 6, 7);
    mfma_agpr_acc<BF16>(dqacc[qb][db], op, __builtin_bit_cast(i16x8, b));
  };

  // ---- VALU slices of two accumulator elements (c = 8 qb + g: elements 2g, 2g+1)
  constexpr int NSL = 8 * QB;
  auto p_slice = [&](int c) __attribute__((always_inline)) {     // P = 2^(c S + c m)
    const int qb = c >> 3, g = c & 7;
    if constexpr (ALIBI) {
      const float r0 = (float)(8 * ((2 * g) >> 2) + ((2 * g) & 3));
      pv[qb][2 * g] = exp2_fast(__builtin_fmaf(sacc[qb][2 * g], c_scale, __builtin_fmaf(b2, r0, lq[qb])));
      pv[qb][2 * g + 1] =
          exp2_fast(__builtin_fmaf(sacc[qb][2 * g + 1], c_scale, __builtin_fmaf(b2, r0 + 1.f, lq[qb])));
    } else {
      pv[qb][2 * g] = exp2_fast(__builtin_fmaf(sacc[qb][2 * g], c_scale, cm[qb]));
      pv[qb][2 * g + 1] = exp2_fast(__builtin_fmaf(sacc[qb][2 * g + 1], c_scale, cm[qb]));
    }
  };
  auto ds_slice = [&](int c) __attribute__((always_inline)) {    // dS = P (dP - delta)
    const int qb = c >> 3, g = c & 7;
    dsk[qb][g] = pack2<BF16>(pv[qb][2 * g] * dpacc[qb][2 * g], pv[qb][2 * g + 1] * dpacc[qb][2 * g + 1]);
  };
  // KPM: padding keys' probabilities -> 0: element i of a lane of half hi holds key
  // 8 (i / 4) + 4 hi + i % 4 of the step
  auto pad_zero = [&](unsigned pad) __attribute__((always_inline)) {
    static_for<16>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      constexpr int k = 8 * (i >> 2) + (i & 3);
      // bit k (lanes 0-31) and bit k + 4 (lanes 32-63), each spread over a half of the lane
      // mask by an arithmetic shift
      const unsigned lo = (unsigned)((int)(pad << (31 - k)) >> 31);
      const unsigned hi = (unsigned)((int)(pad << (27 - k)) >> 31);
      const unsigned long long lanes = (unsigned long long)hi << 32 | lo;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        pv[qb][i] = __builtin_amdgcn_inverse_ballot_w64(lanes) ? 0.f : pv[qb][i];
    });
  };
  // Hidden pairs of band-edge steps are zeroed after P is formed (a branch around VALU only).
  // Keys past the sequence need no mask (their K rows are zero fills, so they add nothing to
  // dQ); queries past it are not stored.  q - key - dlo = u - (8 (i/4) + i%4), u per lane.
  //
  // Where only a lower band edge on a multiple of 32 crosses the step, every 32x32 block is
  // wholly visible, wholly hidden or cut along its diagonal: q - key = x + (column - row) with
  // x = qw0 + 32 qb - k0 a multiple of 32.  Those blocks take constant lane masks.
  // (hide: every pair of the step hidden)
  auto mask_step = [&](int t, bool hide) __attribute__((always_inline)) {
    keep_branch();   // not worth running on every step
    const int k0 = (s_begin + t) * kBK;
    if (hide || ((a.dlo & 31) == 0 && a.dhi - (qw0 + 32 * (QB - 1) - k0) >= 31)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int lo = hide ? 32 : a.dlo - (qw0 + 32 * qb - k0);   // visible iff column - row >= lo
        if (lo >= 32) {
#pragma unroll
          for (int i = 0; i < 16; ++i) pv[qb][i] = 0.f;
        } else if (lo == 0) {
          static_for<16>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            pv[qb][i] = keep_lanes(pv[qb][i], diag_lanes<true>(i));
          });
        }
      }
      return;
    }
    const unsigned span = (unsigned)(a.dhi - a.dlo);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int u = qw0 + 32 * qb + l32 - k0 - 4 * hi - a.dlo;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pv[qb][i] = (unsigned)(u - 8 * (i >> 2) - (i & 3)) <= span ? pv[qb][i] : 0.f;
    }
  };
  auto edge_step = [&](int t) __attribute__((always_inline)) {   // some pair outside the band
    const int k0 = (s_begin + t) * kBK;
    return qw0 - (k0 + kBK - 1) < a.dlo || qw0 + S::QW - 1 - k0 > a.dhi;
  };
  auto pin_p = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) pin(pv[qb]);
  };
  auto pin_ds = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int g = 0; g < 8; ++g) pin(dsk[qb][g]);
  };

  // KPM: the padding word of the current step (scalar, taken in phase 1 once the LDS reads
  // before it have landed) and the next step's as read from LDS
  unsigned pad = 0, pwv = 0;
  // phase 1 of step s: dQ_{s-1}, dP_s | P_s.  P slices start after the second MFMA: S_s was
  // the last product of the step before.  It starts once the K_{s-1}^T halves have landed
  // (the V_s rows may still be in flight) and runs dP_s once they have too.
  // (ek: the entry of step s + kPD, whose tiles it copies)
  auto phase1 = [&](int s, int ek) __attribute__((always_inline)) {
    wait_lgkmcnt_fence<KS>();
    static_for<NG + NM>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m == NG) {
        wait_lgkmcnt_fence<0>();   // V_s rows have landed
        if constexpr (KPM) {       // this step's padding word has too; read the next one's
          pad = __builtin_amdgcn_readfirstlane(pwv);
          pwv = pwords[s + 1 + pw_off];
        }
      }
      if constexpr (m < NG) mfma_dq(std::integral_constant<int, m>{});
      else mfma_dp(std::integral_constant<int, m - NG>{});
      constexpr int W = NG + NM - 2;
      if constexpr (m >= 2) dq_slices<(m - 2) * NSL / W, (m - 1) * NSL / W>(p_slice);
      if constexpr (m >= NG) {
        constexpr int h = m - NG;
        static_for<(h + 1) * NR1 / NM - h * NR1 / NM>([&](auto jc) __attribute__((always_inline)) {
          read_one(std::integral_constant<int, h * NR1 / NM + decltype(jc)::value>{});
        });
      }
      if constexpr (m == 1) copy_tiles(s + kPD, ek);
      __builtin_amdgcn_sched_barrier(0);
    });
    pin_p();
  };
  // phase 2 of step s: S_{s+1} | dS_s; reads the V_{s+1} rows.  It starts once the K_{s+1}
  // rows have landed (the K_s^T halves may still be in flight).  dS slices start after the
  // second MFMA: dP_s was the last product of phase 1.
  auto phase2 = [&]() __attribute__((always_inline)) {
    wait_lgkmcnt_fence<kTrWait>();
    static_for<NM>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      mfma_s(mc);
      constexpr int W = NM - 2;
      if constexpr (m >= 2) dq_slices<(m - 2) * NSL / W, (m - 1) * NSL / W>(ds_slice);
      static_for<(m + 1) * KS / NM - m * KS / NM>([&](auto jc) __attribute__((always_inline)) {
        constexpr int ks = m * KS / NM + decltype(jc)::value;
        va[ks] = __builtin_bit_cast(i16x8, lds_read16_nowait<KTILE>(row_a[ks]));
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    pin_ds();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) keep(ndv[qb]);   // dP's initial value
  };

  // ---- prologue: tiles 0..kPD-1, S_0 and the V_0 rows; dQ_{-1} adds zeros (zero dS and
  // K^T operands)
  static_assert(kPD == 4, "entries of steps 0 .. 3 in h0 .. h3");
  issue_copies(0, h0);
  issue_copies(1, h1);
  issue_copies(2, h2);
  issue_copies(3, h3);
  // Q^T, dO^T, dQ^T and the statistics are used only now: waiting for the Q and dO rows does
  // not hold back the copies, whose latency overlaps theirs
  if (form_stats) {
    // the statistics of the lane's query: m = -LSE / sigma and -delta, zero for a slot past
    // the sequence and for a row that sees no key (LSE = -inf).  The lane holds the 16-byte
    // chunks 2 ks + hi of its rows of O and dO; the two halves of the wave trade their chunk
    // sums and both add all of them in delta_chunk's pairwise order.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float cs[2 * KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const float mine = delta_chunk<BF16>(ov[qb][ks], __builtin_bit_cast(u32x4, greg[qb][ks]));
        const unsigned u = __float_as_uint(mine);
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        cs[2 * ks] = __uint_as_float(r[0]);       // chunk 2 ks, from the lower half
        cs[2 * ks + 1] = __uint_as_float(r[1]);   // chunk 2 ks + 1, from the upper half
      }
#pragma unroll
      for (int w = 1; w < 2 * KS; w *= 2)
#pragma unroll
        for (int i = 0; i < 2 * KS; i += 2 * w) cs[i] += cs[i + w];
      const int q = qw0 + 32 * qb + l32;
      const float lse = lse_in[qb];
      const bool live = q < n && lse != -__builtin_inff();
      lse_in[qb] = live ? -lse / a.sigma : 0.f;
      nd_in[qb] = live ? -cs[0] : 0.f;
      stat_out[qb] = hi ? nd_in[qb] : lse_in[qb];   // stored with dQ, at the end of the tile
    }
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      in_agpr(qreg[qb][ks]);
      in_agpr(greg[qb][ks]);
    }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) in_agpr(dqacc[qb][db]);
  mfma_operand_wait();
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const bool ok = qw0 + 32 * qb + l32 < n;
    cm[qb] = ok ? c_scale * lse_in[qb] : 0.f;
    if constexpr (ALIBI) lq0[qb] = __builtin_fmaf(-b2, (float)(qw0 + 32 * qb + l32 + off - 4 * hi), cm[qb]);
    const float nd = ok ? nd_in[qb] : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ndv[qb][i] = nd;
  }
  wait_vmcnt<0>();
  wg_barrier();
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int g = 0; g < 8; ++g) dsk[qb][g] = 0u;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      kt_lo[kk][db] = kt_hi[kk][db] = i16x4{};
      pin(kt_lo[kk][db]);              // zeros held in the operand registers (not rematerialised
      pin(kt_hi[kk][db]);              // by a VALU write right before the first product)
    }
  read_rows(row_a, Z{}, ka);           // K_0
  read_rows(row_a, KT{}, va);          // V_0
  wait_lgkmcnt0_fence();
  if (TS > 0) static_for<NM>([&](auto mc) __attribute__((always_inline)) { mfma_s(mc); });
  pin_ds();
  mfma_result_wait();   // S_0 is read by VALU in step 0
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) pin(sacc[qb]);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) row_a[ks] += stage_step(0);   // rows: tile 1

  if constexpr (KPM) pwv = pwords[pw_off];   // (landed by step 0's phase-1 fence)
  // ---- steps: one barrier each
  for (int s = 0; s < TS; ++s) {
    if constexpr (ALIBI) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) lq[qb] = __builtin_fmaf(b2, (float)((s_begin + s) * kBK), lq0[qb]);
    }
    int ek = s + kPD, es = s;
    if constexpr (BLK) {
      if (((s + kPD) & 63) == 0) win = list[s + kPD + lane];   // the next window (rare)
      ek = __builtin_amdgcn_readlane(win, (s + kPD) & 63);
      es = h0;
      h0 = h1;
      h1 = h2;
      h2 = h3;
      h3 = ek;
    }
    phase1(s, ek);
    const bool hide = BLK && !entry_selected(es, wave >> 1);
    const bool ed = edge_step(rel(es));
    if (hide || ed || pad != 0) {
      if (hide || ed) mask_step(rel(es), hide);
      if constexpr (KPM) pad_zero(pad);
      pin_p();
    }
    phase2();
    // next stage: rows move to tile s+2, transposed halves to tile s+1
    {
      const int d0 = stage_step(s), d1 = stage_step(s + 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) row_a[ks] += d1;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < DB; ++db) tr_a[h][db] += d0;
    }
    wait_vmcnt<(kPD - 2) * 2 * CPT>();
    wg_barrier();
  }
  wait_lgkmcnt0_fence();
  // dQ of the last step
  if (TS > 0) {
    static_for<NG>([&](auto mc) __attribute__((always_inline)) {
      mfma_dq(mc);
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  wait_vmcnt<0>();   // no copy may land after the workgroup ends

  // ---- epilogue: lane holds query qw0 + 32 qb + l32, dims 32 db + 8 g + 4 hi + 0..3
  // The statistics block of each of the wave's 32-query blocks (slots past the sequence
  // included), stored here rather than in the prologue, whose final wait would hold the
  // workgroup for the store's completion.
  if (form_stats) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      if (qw0 + 32 * qb < nr) a.stats_out[stat_index(bh, nr, qw0 + 32 * qb + l32) + hi * kStatRows] = stat_out[qb];
  }
  mfma_result_wait();
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) in_agpr(dqacc[qb][db]);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qw0 + 32 * qb + l32;
    if (q < (PADDED ? nw : n)) {
      char* row = a.dq + head + (long)q * RB;
      const float sc = a.scale;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dim = 32 * db + 8 * g + 4 * hi;
          u32x2 w = {pack2<BF16>(dqacc[qb][db][4 * g + 0] * sc, dqacc[qb][db][4 * g + 1] * sc),
                     pack2<BF16>(dqacc[qb][db][4 * g + 2] * sc, dqacc[qb][db][4 * g + 3] * sc)};
          if (PADDED && q >= n) w = u32x2{};   // padding rows: zero gradients
          *reinterpret_cast<u32x2*>(row + dim * 2) = w;
        }
    }
  }
}

// Under a causal mask (no left window) the number of key steps grows linearly with the query
// tile: paired as t and n_tiles - 1 - t, the workgroups are of equal length.  Unpaired, the
// latest (longest) tiles go first.
// PADDED: a padded batch (per-batch lengths), a separate instance
template <int D, bool BF16, bool PADDED, bool ALIBI = false, bool BLK = false, bool KPM = false>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void dq_main_kernel(DqArgs a) {
  constexpr int kExtra = BLK ? block_list_bytes<2>() : KPM ? 4 * (kListMax + 64) + 16 : 0;
  __shared__ __attribute__((aligned(1024))) char lds_raw[kNS * QShape<D>::STAGE + kExtra];
  char FA_LDS* ring = (char FA_LDS*)lds_raw;
  int FA_LDS* list = (int FA_LDS*)(lds_raw + kNS * QShape<D>::STAGE);
  int bh, t;
  xcd_tile_order(blockIdx.x, a.n_bh, a.n_units, bh, t);
  t = a.n_tiles - 1 - t;
  const int n_pass = a.paired && t != a.n_tiles - 1 - t ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
    if (pass > 0) wg_barrier();   // every wave is done with the ring before it is refilled
    dq_tile<D, BF16, PADDED, ALIBI, BLK, KPM>(a, ring, list, bh, pass == 0 ? t : a.n_tiles - 1 - t);
  }
}

// nq query rows over nk key rows (dense operands); query i at key position i + nk - nq
template <int D, bool BF16>
hipError_t launch(const BwdParams& p, int nq, int nk, hipStream_t stream, bool form_stats = false) {
  using S = QShape<D>;
  DqArgs a;
  a.q = static_cast<const char*>(p.q);
  a.k = static_cast<const char*>(p.k);
  a.v = static_cast<const char*>(p.v);
  a.dout = static_cast<const char*>(p.dout);
  a.stats = p.stats;
  a.stats_out = form_stats ? p.stats : nullptr;
  a.o = static_cast<const char*>(p.o);
  a.lse = p.lse;
  a.sigma = softmax_sigma(p.scale);
  a.dq = static_cast<char*>(p.dq);
  a.seqlens = p.seqlens;
  a.cu = p.cu;
  a.total = p.total;
  a.n = nq;
  a.nk = nk;
  a.off = nk - nq;
  a.heads = p.H;
  a.n_bh = p.B * p.H;
  a.n_tiles = (nq + S::QWG - 1) / S::QWG;
  a.c = (float)((double)softmax_sigma(p.scale) * 1.4426950408889634);
  a.scale = p.scale;
  a.causal = p.causal;
  a.wl = p.window_left;
  a.wr = p.causal ? 0 : p.window_right;
  // a window of kUnbounded or more is no bound (see the dK/dV kernel)
  constexpr int kUnbounded = 1 << 30;
  const int wr = p.window_right < 0 ? kUnbounded : std::min(p.window_right, kUnbounded);
  const int wl = p.window_left < 0 ? kUnbounded : std::min(p.window_left, kUnbounded);
  // the band in query-index space: positions are indices + nk - nq
  a.dlo = (p.causal ? 0 : -wr) - (nk - nq);
  a.dhi = wl - (nk - nq);
  const int half = (a.n_tiles + 1) / 2;
  // pair only where the visible key count of the last query tile is at least twice that of
  // the first (see the forward): not for a short block of queries over a long cache
  a.paired = p.causal && p.window_left < 0 && nq >= (nk - nq) + 2 * S::QWG &&
             (long)a.n_bh * half >= 256;
  a.n_units = a.paired ? half : a.n_tiles;
  a.slopes = p.slopes;
  a.blocks = p.blocks;
  a.kpm = p.kpm;
  a.n_qb = (nq + 63) / 64;
  a.n_kb = (nk + 63) / 64;
  const long blocks = (long)a.n_bh * a.n_units;
  if (p.slopes != nullptr)   // (no padded batch takes ALiBi or a block mask)
    hipLaunchKernelGGL((dq_main_kernel<D, BF16, false, true>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, a);
  else if (p.blocks != nullptr)
    hipLaunchKernelGGL((dq_main_kernel<D, BF16, false, false, true>), dim3((unsigned)blocks), dim3(kThreads),
                       0, stream, a);
  else if (p.kpm != nullptr)
    hipLaunchKernelGGL((dq_main_kernel<D, BF16, false, false, false, true>), dim3((unsigned)blocks),
                       dim3(kThreads), 0, stream, a);
  else if (p.seqlens != nullptr || p.cu != nullptr)
    hipLaunchKernelGGL((dq_main_kernel<D, BF16, true>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((dq_main_kernel<D, BF16, false>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dq_main(const BwdParams& p, hipStream_t stream, bool form_stats) {
  if (p.D == 64)
    return p.bf16 ? launch<64, true>(p, p.N, p.N, stream, form_stats)
                  : launch<64, false>(p, p.N, p.N, stream, form_stats);
  return p.bf16 ? launch<128, true>(p, p.N, p.N, stream, form_stats)
                : launch<128, false>(p, p.N, p.N, stream, form_stats);
}

hipError_t launch_dq_main_kv(const BwdParams& p, int nq, int nk, hipStream_t stream, bool form_stats) {
  if (p.D == 64)
    return p.bf16 ? launch<64, true>(p, nq, nk, stream, form_stats) : launch<64, false>(p, nq, nk, stream, form_stats);
  return p.bf16 ? launch<128, true>(p, nq, nk, stream, form_stats)
                : launch<128, false>(p, nq, nk, stream, form_stats);
}

}  // namespace fa
