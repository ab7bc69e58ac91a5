// Fused attention forward for gfx950: the kernel for grids that fill the chip.
//
// A workgroup of 4 waves owns tiles of 128 query rows of one (batch, head), 32 rows per
// wave; two workgroups share a CU, so each SIMD runs one wave of each.  The two waves of a
// SIMD then meet no common barrier, and neither idles while the other finishes a step.  The
// key/value sequence is processed in tiles of BC keys (64 for head dim 64, 32 for 128).  Per
// key tile j each wave does
//
//   GEMM0  S_j^T = K_j Q^T                  MFMA 32x32x16, Q^T in registers, K from LDS
//   ALU0   row max of S_j, reference update, x = s*c - m                  (VALU)
//   ALU1   P_j = 2^x, row sum l += P_j, P_j rounded to the input type     (VALU, exp)
//   GEMM1  O^T += V_j^T P_j^T               MFMA, V^T read from LDS transposed, P^T taken
//                                           straight from the S^T accumulators' registers
//
// Computing the transposed score block puts one query in each lane (keys spread over the
// lane's registers and its partner lane l^32), so row max and row sum are in-lane
// reductions plus one permlane32 swap, and rescaling O^T is a per-lane scalar multiply.
//
// The loop is software-pipelined in two phases per key tile, with the score registers
// double buffered (S_{j+1} is produced while P_j is being formed):
//
//   phase 1  GEMM0_{j+1} interleaved with ALU1_j and the reads of the V_j operands
//            (LDS -> registers, landing under the compute)
//   phase 2  edge mask of S_{j+1}; GEMM1_j interleaved with ALU0_{j+1} and the reads of the
//            K_{j+2} operands; O rescaled where a reference moved
//
// Scheduling barriers interleave each phase's MFMAs with its VALU work and operand reads, and
// empty asm statements keep each phase's VALU results from being sunk into the next phase.
// K and V tiles arrive by direct global->LDS copies (no registers, no LDS write
// instructions) into rings of kNS stages, issued kPD tiles ahead; the 16-byte chunks are
// placed so that the LDS layout is the XOR-swizzled one the operand reads expect (no bank
// conflicts).  The loop is unrolled over the ring stages, so every operand address is a
// register plus an immediate.  One workgroup barrier per key tile publishes the copies and
// guards ring reuse.
//
// Under a causal mask with no left window bound the work of a query tile grows with its
// index; there a workgroup processes two query tiles, qt and n_qt - 1 - qt, so that every
// workgroup has the same amount of work (when that still leaves a workgroup per CU).  Every
// wave computes every key tile the workgroup visits; tiles hidden from some or all of a
// wave's queries go through the mask and contribute P = 0.
//
// The arithmetic follows the tiling of "告别OOM和训练慢：用Flash Attention加速你的PyTorch大模型
// （含A100环境配置）" §2.1 with the running max / running sum of its §2.2 (read as
// l_new = exp(m_old - m_new) l_old + sum exp(s - m_new), O rescaled by the same factor and
// divided by l once at the end), one query block against all visible key blocks as "Flash
// Attention 3.7 核心原理与实战：加速Transformer模型训练与推理" §3.1 describes.  The reference m of a
// row is the exact maximum of its first visible tile and moves to a later tile's exact
// maximum when that one is not negligible against the mass already summed (2^g * 16 > l) or
// exceeds m by more than kTau (base-2 units); the softmax does not depend on the shift (the safe-softmax
// argument of the same §2.2), rows dominated by a few keys keep a largest probability of
// exactly 1, and probabilities stay below 2^kTau.  l is summed in fp32 from unrounded
// probabilities; P is rounded once to the input type; LSE = ln 2 * (m + log2 l).
#include <cmath>
#include <type_traits>

#include "block_list.h"
#include "cdna4.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kWaves = 4;          // one per SIMD: two workgroups share a CU
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;   // query rows per query tile (32 per wave)
constexpr int kPD = 3;             // key tiles copied ahead
constexpr int kNS = kPD + 1;       // LDS ring stages, K and V each (the loop is unrolled over them)
constexpr float kTau = 8.0f;
constexpr float kNoRef = -1e30f;   // reference of a row with no visible key yet

struct MainArgs {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  const int* seqlens;   // per-batch lengths (device, may be null: every sequence has n rows)
  const int* cu;        // packed batch: per-batch start rows [B + 1] (device), or null
  int total;            // packed batch: rows per head (the concatenated sequences)
  int n;          // query rows per (batch, head): the sequence length, or the padded one with seqlens
  int nk;         // key rows per (batch, head) (n for self-attention and padded batches)
  int off;        // key position of query 0 (nk - n; 0 for padded batches)
  int heads;
  int n_bh;       // batch * heads
  int n_qt;       // query tiles per head
  int n_units;    // workgroups per head: n_qt, or ceil(n_qt / 2) query-tile pairs
  int paired;     // a workgroup takes query tiles u and n_qt - 1 - u
  float c;        // max(|softmax_scale|, tiny) * log2(e)
  unsigned q_sign;  // 0x80008000 negates Q (negative scale)
  int causal, wl, wr;
  const float* slopes;  // ALiBi slopes [heads] (device), read by the ALIBI instances only
  const unsigned char* blocks;   // BLK: block-sparse mask [heads][n_qb][n_kb] of 64 x 64 blocks
  int n_qb, n_kb;
  const unsigned char* kpm;      // KPM: key padding mask [batch][nk] (nonzero = padding key)
};

template <int D>
struct Shape {
  static constexpr int BC = D == 64 ? 64 : 32;   // keys per tile
  static constexpr int MB = BC / 32;             // 32-key blocks of S^T
  static constexpr int KS = D / 16;              // k-steps of Q K^T
  static constexpr int DB = D / 32;              // 32-dim blocks of O^T
  static constexpr int KK = BC / 16;             // 16-key steps of P V
  static constexpr int RB = D * 2;               // bytes per row
  static constexpr int TILE = BC * RB;           // bytes per K or V tile
  static constexpr int CPT = TILE / (16 * kThreads);   // 16-byte copies per thread per tile
  static_assert(CPT * 16 * kThreads == TILE, "whole 16-byte chunks per thread");
  static_assert(kPD >= 2, "the phase-1 wait keeps one iteration of copies in flight");
  static_assert((kNS - 1) * TILE + (KK - 1) * 16 * RB < 65536 &&
                (kNS - 1) * TILE + (MB - 1) * 32 * RB < 65536, "operand offsets fit the ds immediate");
};

// PADDED: a padded batch (per-batch lengths); a separate instance, so that the plain one
// carries none of its code.
// ALIBI: every score gets the ALiBi penalty -slope_h |p - j| (p the query's key position, j the
// key's), in the exponent domain: y = s c - slope log2(e) |p - j|.  The row statistics are
// taken over y, so y is formed before the row maximum, relative to the row's current reference
// (0 before its first visible tile), and moved to a new reference only where one is set.
// BLK: a block-sparse mask.  A query tile's two 64-query blocks select key tiles; the
// workgroup visits only the tiles one of them selects (a list of them in LDS, built at the
// start of the tile), and a wave whose block does not select a visited tile sees it hidden.
// KPM: a key padding mask.  At the start of a query tile the workgroup gathers one padding
// word per key tile (bit k: key k of the tile is padding) into LDS and drops the leading and
// trailing tiles made only of padding; a tile with some padding sets those keys' scores to
// -inf, one v_cndmask per score with a scalar lane mask (the keys of a score register are the
// same in every lane of a half-wave).
template <int D, bool BF16, bool PADDED, bool ALIBI = false, bool BLK = false, bool KPM = false>
__global__ __launch_bounds__(kThreads, 8 / kWaves) void fwd_main_kernel(MainArgs a) {
  using S = Shape<D>;
  constexpr int BC = S::BC, MB = S::MB, KS = S::KS, DB = S::DB, KK = S::KK, RB = S::RB;
  constexpr int TILE = S::TILE, CPT = S::CPT;

  static_assert(!(ALIBI && BLK), "no instance takes both");
  static_assert(!(KPM && (ALIBI || BLK || PADDED)), "key padding alone");
  constexpr int kExtra = BLK ? block_list_bytes<2>() : KPM ? 8 * kListMax + 16 : 0;
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * kNS * TILE + kExtra];
  char FA_LDS* kring = (char FA_LDS*)lds_raw;
  char FA_LDS* vring = kring + kNS * TILE;
  // BLK: the key tiles the query tile's two 64-query blocks select (block_list.h)
  int FA_LDS* tlist = (int FA_LDS*)(lds_raw + 2 * kNS * TILE);
  // KPM: the padding word of each key tile, then the first and past-last tiles with a key
  unsigned long long FA_LDS* pwords = (unsigned long long FA_LDS*)(lds_raw + 2 * kNS * TILE);
  int FA_LDS* ptrim = (int FA_LDS*)(pwords + kListMax);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, unit;
  xcd_tile_order(blockIdx.x, a.n_bh, a.n_units, bh, unit);
  // rows of the head in memory (nr) and of its sequence (n); rows n .. nr-1 are padding, read
  // as zeros through the buffer resources and written as zeros (a padded batch).  A packed
  // batch has no padding rows: sequence b is rows cu[b] .. cu[b+1]-1 of each head's `total`
  // concatenated rows (offsets clamped to [0, total], at most nr rows), and nothing past its
  // own rows is written.
  const int nr = a.n;
  int n = nr, nw = nr;   // sequence rows, rows written
  long head = (long)bh * nr * RB, lrow = (long)bh * nr;   // first byte of Q / O, first LSE index
  if constexpr (PADDED) {
    const int b = bh / a.heads, h = bh - b * a.heads;
    if (a.cu != nullptr) {
      const int c0 = min(max(a.cu[b], 0), a.total);
      const int c1 = min(max(a.cu[b + 1], c0), a.total);
      n = nw = min(c1 - c0, nr);
      lrow = (long)h * a.total + c0;
      head = lrow * RB;
    } else {
      n = min(max(a.seqlens[b], 0), nr);
    }
  }
  // keys: a padded batch has as many as queries; otherwise nk rows, query i at position i + off
  const int nkr = PADDED ? n : a.nk;
  const int off = PADDED ? 0 : a.off;
  const long khead = PADDED ? head : (long)bh * a.nk * RB;
  const int head_bytes = nkr * RB;   // K and V bytes of the head's keys
  const auto rq = make_rsrc(a.q + head, n * RB);
  const auto rk = make_rsrc(a.k + khead, head_bytes);
  const auto rv = make_rsrc(a.v + khead, head_bytes);
  const Mask mk{nkr, a.causal, a.wl, a.wr};
  const float c = a.c;
  const float NEG_INF = -__builtin_inff();
  const float b2 = ALIBI ? a.slopes[bh % a.heads] * kLog2e : 0.f;   // ALiBi slope, base 2

  // With 8 waves, the two waves of a SIMD (w and w + 4) own neighbouring 32-row stripes, so
  // under a causal mask they have nearly the same number of visible keys.
  const int stripe = kWaves == 8 ? 2 * (wave & 3) + (wave >> 2) : wave;

  // ---- per-lane constants
  // transposing-read coordinates (see cdna4.h): 16-lane group, row, quad
  const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
  const int tr_key = (tg >> 1) * 4 + tr;
  const int tr_byte = (tq & 1) * 8;
  // LDS addresses of the operands in ring stage 0; stage st, the 32-key block mb (K) and the
  // 16-key step kk (V) add immediate offsets (st TILE, 32 mb RB, 16 kk RB): the swizzle of a
  // row depends only on bits that adding 16 or 32 rows leaves alone.  K operand of k-step ks:
  // row l32, chunk 2 ks + hi.  V^T operand half h of dim block db: rows tr_key + 8 h.
  unsigned ka[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) ka[ks] = lds_addr(kring) + tile_offset<D>(l32, 2 * ks + hi);
  unsigned va[2][DB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      va[h][db] = lds_addr(vring) + tile_offset<D>(tr_key + 8 * h, 4 * db + 2 * (tg & 1) + (tq >> 1)) + tr_byte;
  // async copies: thread tid fills physical 16-byte chunks tid + kThreads j of each tile;
  // chunk tid + kThreads j lies 16 kThreads j / RB rows below chunk tid, which keeps its swizzle
  const int cp_row = (16 * tid) / RB;
  const int cp_src = cp_row * RB + ((((16 * tid) % RB) / 16) ^ chunk_swizzle<D>(cp_row)) * 16;

  const int npass = (a.paired && a.n_qt - 1 - unit != unit) ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
    const int qt = a.paired ? (pass == 0 ? a.n_qt - 1 - unit : unit) : unit;
    if (pass > 0) wg_barrier();      // the previous tile's last LDS reads are done

    const int q0 = qt * kBr;
    const int wq0 = q0 + 32 * stripe;
    const int qi = wq0 + l32;
    if (PADDED && q0 >= n) {   // padding rows only: O = 0, LSE = -inf
      if (qi < nw) {
        char* orow = a.o + head + (long)qi * RB;
#pragma unroll
        for (int c16 = 0; c16 < RB / 32; ++c16)
          *reinterpret_cast<u32x4*>(orow + 32 * c16 + 16 * hi) = u32x4{};
        if (a.lse != nullptr && hi == 0) a.lse[lrow + qi] = NEG_INF;
      }
      continue;
    }

    // Q^T operands, read once (B operand of every S^T product)
    i16x8 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = buffer_load16(rq, qi * RB + (2 * ks + hi) * 16);
      x ^= a.q_sign;
      qreg[ks] = __builtin_bit_cast(i16x8, x);
    }

    int key_lo, key_hi;
    mk.key_range(q0 + off, min(q0 + kBr - 1, n - 1) + off, key_lo, key_hi);
    if (key_hi <= key_lo) {   // no query of the tile sees a key (only with fewer keys): O = 0
      if (qi < n) {
        char* orow = a.o + head + (long)qi * RB;
#pragma unroll
        for (int c16 = 0; c16 < RB / 32; ++c16)
          *reinterpret_cast<u32x4*>(orow + 32 * c16 + 16 * hi) = u32x4{};
        if (a.lse != nullptr && hi == 0) a.lse[lrow + qi] = NEG_INF;
      }
      continue;
    }
    int t_begin = key_lo / BC;
    int T = (key_hi + BC - 1) / BC - t_begin;   // key tiles the workgroup visits (>= 1)
    int pw_off = 0;                             // KPM: padding word of tile t at pwords[t + pw_off]
    if constexpr (KPM) {
      const unsigned char* kp = a.kpm + (long)(bh / a.heads) * nkr;
      for (int t = wave; t < T; t += kWaves) {
        const int j = (t_begin + t) * BC + lane;
        const bool pad = lane >= BC || j >= nkr || kp[j] != 0;
        const unsigned long long w = __ballot(pad);
        if (lane == 0) pwords[t] = w;
      }
      wait_lgkmcnt0();   // (the barrier does not wait for LDS writes)
      wg_barrier();
      if (wave == 0) {
        int first = T, last = -1;
        for (int c = 0; c < T; c += 64) {
          const bool live = c + lane < T && pwords[c + lane] != ~0ull;
          const unsigned long long b = __ballot(live);
          if (b != 0) {
            if (first == T) first = c + __builtin_ctzll(b);
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
      if (past <= first) {   // every key of the tile's range is padding: O = 0, LSE = -inf
        if (qi < n) {
          char* orow = a.o + head + (long)qi * RB;
#pragma unroll
          for (int c16 = 0; c16 < RB / 32; ++c16)
            *reinterpret_cast<u32x4*>(orow + 32 * c16 + 16 * hi) = u32x4{};
          if (a.lse != nullptr && hi == 0) a.lse[lrow + qi] = NEG_INF;
        }
        continue;
      }
      t_begin += first;
      T = past - first;
      pw_off = first;
    }
    // BLK: the selected tiles among those T, listed in LDS; TT tiles run through the pipeline
    int TT = T;
    if constexpr (BLK) {
      TT = build_block_list<2, BC, kPD + 2, kWaves>(tlist, a.blocks + (long)(bh % a.heads) * a.n_qb * a.n_kb,
                                                    a.n_kb, 1, q0 >> 6, a.n_qb, t_begin, T, lane, wave);
      if (TT == 0) {   // no selected tile: O = 0, LSE = -inf
        if (qi < n) {
          char* orow = a.o + head + (long)qi * RB;
#pragma unroll
          for (int c16 = 0; c16 < RB / 32; ++c16)
            *reinterpret_cast<u32x4*>(orow + 32 * c16 + 16 * hi) = u32x4{};
          if (a.lse != nullptr && hi == 0) a.lse[lrow + qi] = NEG_INF;
        }
        continue;
      }
    }
    // pipeline step k -> the tile it runs (BLK: list entry; else the index itself) and its
    // index after t_begin
    auto ent = [&](int k) __attribute__((always_inline)) {
      if constexpr (BLK) return __builtin_amdgcn_readfirstlane(tlist[k]);
      else return k;
    };
    auto rel = [&](int e) __attribute__((always_inline)) { return BLK ? entry_step(e) : e; };
    // BLK: the entries of steps i + 1 .. i + 3 of iteration i (scalars, shifted along), and the
    // one of step i + kPD + 1, read from LDS one iteration ahead
    int h1 = 0, h2 = 0, h3 = 0, pre = 0;
    if constexpr (BLK) {
      h1 = ent(1);
      h2 = ent(2);
      h3 = ent(3);
      pre = tlist[4];
    }
    // visible key interval of this lane's query (edge tiles), from its key position; a query
    // that sees no key gets an interval past every key
    const int qpos = qi + off;
    int row_lo = mk.wl >= 0 ? max(0, qpos - mk.wl) : 0;
    int row_hi = min(nkr - 1, mk.causal ? qpos : (mk.wr >= 0 ? qpos + mk.wr : nkr - 1));
    if (row_hi < row_lo) row_lo = row_hi = nkr + 2 * BC;

    // ring stage of a tile is its index mod kNS; ST is that stage where the caller knows it
    // (ek, ev: the entries of the K and V tiles, see ent)
    auto issue_copies = [&](int ek, int ev, int st_k, int st_v) __attribute__((always_inline)) {
      // tiles past the last one read beyond the buffer: zero fills, no memory traffic
      const int tk = rel(ek), tv = rel(ev);
      const int ok = tk < T ? (t_begin + tk) * TILE : head_bytes;
      const int ov = tv < T ? (t_begin + tv) * TILE : head_bytes;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        buffer_load16_lds(rk, kring + st_k * TILE + 16 * kThreads * j + 1024 * wave, cp_src + 16 * kThreads * j + ok);
        buffer_load16_lds(rv, vring + st_v * TILE + 16 * kThreads * j + 1024 * wave, cp_src + 16 * kThreads * j + ov);
      }
    };

    // ---- per-wave state of this query tile
    f32x16 oacc[DB];                 // O^T
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m_ref = kNoRef, m_prev = kNoRef, l_run = 0.f;
    bool moved = false;
    f32x16 sb[2][MB];
    unsigned pk[MB][8];
    u32x4 kop[MB][KS];
    // V^T operands as the two halves the transposing reads return, joined where the MFMA
    // uses them (after the wait), so no copy of them can run before the data has landed
    i16x4 vlo[KK][DB], vhi[KK][DB];

    // Key tiles t_in_lo <= t <= t_in_hi show every key to every query of this wave (the
    // conditions of Mask::all_visible solved for the tile index once, so that the per-tile
    // test is two scalar compares).  Shifts by log2(BC) are floor divisions, also below 0.
    constexpr int SH = BC == 64 ? 6 : 5;
    static_assert((1 << SH) == BC, "tile width is a power of two");
    const int wp0 = wq0 + off;                                          // key position of wq0
    int t_in_hi = (nkr >> SH) - 1;                                        // j1 <= n
    if (mk.causal) t_in_hi = min(t_in_hi, (wp0 - BC + 1) >> SH);        // j1 - 1 <= q_first
    if (mk.wr >= 0) t_in_hi = min(t_in_hi, (wp0 + mk.wr - BC + 1) >> SH);
    const int t_in_lo = (mk.wl >= 0 ? -((mk.wl - wp0 - 31) >> SH) : 0) - t_begin;  // j0 >= q_last - wl
    t_in_hi -= t_begin;
    auto edge = [&](int t) __attribute__((always_inline)) {
      return t < t_in_lo || t > t_in_hi;
    };

    // ---- the pieces of work.  Operand reads are untracked (waited for with lgkmcnt fences);
    // ST is the ring stage as a constant, so every address is a register plus an immediate.
    auto read_k = [&](auto stc) __attribute__((always_inline)) {
      constexpr int ST = decltype(stc)::value;
      static_for<KS>([&](auto ksc) __attribute__((always_inline)) {
        constexpr int ks = decltype(ksc)::value;
        static_for<MB>([&](auto mbc) __attribute__((always_inline)) {
          constexpr int mb = decltype(mbc)::value;
          kop[mb][ks] = lds_read16_nowait<ST * TILE + 32 * mb * RB>(ka[ks]);
        });
      });
    };
    auto read_v = [&](auto stc) __attribute__((always_inline)) {
      constexpr int ST = decltype(stc)::value;
      static_for<KK>([&](auto kkc) __attribute__((always_inline)) {
        constexpr int kk = decltype(kkc)::value;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          vlo[kk][db] = lds_read_tr_nowait<ST * TILE + kk * 16 * RB>(va[0][db]);
          vhi[kk][db] = lds_read_tr_nowait<ST * TILE + kk * 16 * RB>(va[1][db]);
        }
      });
    };
    // single operand reads by flat index, for spreading them over a phase's MFMA slots
    auto read_k_one = [&](auto stc, auto fc) __attribute__((always_inline)) {
      constexpr int ST = decltype(stc)::value, f = decltype(fc)::value, ks = f / MB, mb = f % MB;
      kop[mb][ks] = lds_read16_nowait<ST * TILE + 32 * mb * RB>(ka[ks]);
    };
    auto read_v_one = [&](auto stc, auto fc) __attribute__((always_inline)) {
      constexpr int ST = decltype(stc)::value, f = decltype(fc)::value;
      constexpr int kk = f / (2 * DB), db = (f / 2) % DB, h = f % 2;
      if constexpr (h == 0)
        vlo[kk][db] = lds_read_tr_nowait<ST * TILE + kk * 16 * RB>(va[0][db]);
      else
        vhi[kk][db] = lds_read_tr_nowait<ST * TILE + kk * 16 * RB>(va[1][db]);
    };
    // V^T * P^T products of one 16-key step into O^T
    auto pv = [&](auto ec) __attribute__((always_inline)) {
      constexpr int e = decltype(ec)::value, kk = e / DB, db = e % DB;
      const u32x4 pb = {pk[kk >> 1][4 * (kk & 1) + 0], pk[kk >> 1][4 * (kk & 1) + 1],
                        pk[kk >> 1][4 * (kk & 1) + 2], pk[kk >> 1][4 * (kk & 1) + 3]};
      oacc[db] = mfma32x32x16<BF16>(__builtin_shufflevector(vlo[kk][db], vhi[kk][db], 0, 1, 2, 3, 4, 5, 6, 7),
                                    __builtin_bit_cast(i16x8, pb), oacc[db]);
    };
    // K Q^T product e of S^T (k-step e / MB, 32-key block e % MB)
    auto qk = [&](auto xb, auto ec) __attribute__((always_inline)) {
      constexpr int X = decltype(xb)::value, e = decltype(ec)::value, ks = e / MB, mb = e % MB;
      sb[X][mb] = mfma32x32x16<BF16>(__builtin_bit_cast(i16x8, kop[mb][ks]), qreg[ks],
                                     ks == 0 ? f32x16{} : sb[X][mb]);
    };
    // hidden scores -> -inf (edge tiles only): key j is visible iff j - row_lo, as an unsigned
    // number, is at most row_hi - row_lo.
    //
    // Where the band's edges lie on multiples of 32 (causal, windows of multiples of 32) and the
    // tile holds no key past the sequence, each 32x32 block is wholly visible, wholly hidden or
    // cut along its diagonal by an edge: q - key = x + (column - row), x = wq0 - (first key of
    // the block) a multiple of 32, column - row in [-31, 31].  Those blocks take constant lane
    // masks instead of compares.
    const bool has_lo = mk.causal || mk.wr >= 0, has_hi = mk.wl >= 0;
    const int d_lo = mk.causal ? 0 : mk.wr >= 0 ? -mk.wr : 0;   // q - key >= d_lo (has_lo)
    const bool band32 = (!has_lo || (d_lo & 31) == 0) && (!has_hi || (mk.wl & 31) == 0) &&
                        (off & 31) == 0;
    // (hide: every score of the tile -> -inf)
    auto mask = [&](auto xb, int t, bool hide) __attribute__((always_inline)) {
      constexpr int X = decltype(xb)::value;
      if (hide || (band32 && (t_begin + t + 1) * BC <= nkr)) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int x = wp0 - ((t_begin + t) * BC + 32 * mb);   // wave-uniform
          const int lo = hide ? 32 : has_lo ? d_lo - x : -32, up = has_hi ? mk.wl - x : 32;
          if (lo >= 32 || up <= -32) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sb[X][mb][r] = NEG_INF;
            continue;
          }
          if (lo == 0)   // column >= row
            static_for<16>([&](auto rc) __attribute__((always_inline)) {
              constexpr int r = decltype(rc)::value;
              sb[X][mb][r] = __builtin_amdgcn_inverse_ballot_w64(diag_lanes<true>(r)) ? sb[X][mb][r] : NEG_INF;
            });
          if (up == 0)   // row >= column
            static_for<16>([&](auto rc) __attribute__((always_inline)) {
              constexpr int r = decltype(rc)::value;
              sb[X][mb][r] = __builtin_amdgcn_inverse_ballot_w64(diag_lanes<false>(r)) ? sb[X][mb][r] : NEG_INF;
            });
        }
        return;
      }
      const unsigned u0 = (unsigned)((t_begin + t) * BC + 4 * hi - row_lo);
      const unsigned width = (unsigned)(row_hi - row_lo);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const unsigned u = u0 + (unsigned)(32 * mb + 8 * (r >> 2) + (r & 3));
          sb[X][mb][r] = u <= width ? sb[X][mb][r] : NEG_INF;
        }
    };
    // ALU0 of S_X: row max, reference update, x = s*c - m (in place)
    // running row max over elements [LO, HI) (LO == 0 starts it)
    auto row_max = [&](auto xb, auto lo_c, auto hi_c, float& ext) __attribute__((always_inline)) {
      constexpr int X = decltype(xb)::value, LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
      if constexpr (LO == 0) ext = sb[X][0][0];
#pragma unroll
      for (int e = LO == 0 ? 1 : LO; e < HI; ++e) ext = fmaxf(ext, sb[X][e / 16][e % 16]);
    };
    auto update_ref = [&](float ext) __attribute__((always_inline)) {
      ext = max_with_partner(ext);
      const float m_tile = ext * c;                     // -inf when no key of the tile shows
      const float g = m_tile - m_ref;                   // +huge on a row's first visible tile
      const float l_row = sum_with_partner(l_run);      // both lanes of a row decide alike
      const bool heavy = exp2_fast(g + 4.f) > l_row;
      const bool move = (g > 0.f) & ((g > kTau) | heavy);
      m_prev = m_ref;
      m_ref = move ? m_tile : m_ref;
      moved = move;
    };
    auto shift = [&](auto xb, auto lo_c, auto hi_c) __attribute__((always_inline)) {
      constexpr int X = decltype(xb)::value, LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
      const float neg_m = -m_ref;
#pragma unroll
      for (int e = LO; e < HI; ++e) sb[X][e / 16][e % 16] = __builtin_fmaf(sb[X][e / 16][e % 16], c, neg_m);
    };
    // ALIBI: y = s c - b2 |p - j| - base, base the row's reference (0 while it has none).  In key
    // tile t (keys j0 ..), element (mb, r) holds key j = j0 + 4 hi + Jr, Jr = 32 mb + 8 (r / 4) +
    // r % 4; with Pl = p - j0 - 4 hi, p - j = Pl - Jr.  Where every key of the tile lies at or
    // before every query of the wave (B = b2), or at or after every one (B = -b2), the penalty is
    // linear in Jr: y = s C + (B Jr + L) with C = c, L = -B Pl - base, two instructions per score
    // with wave-uniform C and B.  Under a causal mask the keys past a query are hidden anyway, so
    // every tile takes B = b2.  A tile around the diagonal of a non-causal call gets
    // s c - b2 |p - j| beforehand (the rare branch), and then C = 1, B = 0, L = -base.
    auto alibi_base = [&]() __attribute__((always_inline)) { return m_ref == kNoRef ? 0.f : m_ref; };
    auto alibi_pl = [&](int t) __attribute__((always_inline)) {
      return (float)(qpos - (t_begin + t) * BC - 4 * hi);
    };
    auto alibi_straddle = [&](int t) __attribute__((always_inline)) {
      const int j0 = (t_begin + t) * BC;
      return !mk.causal && j0 + BC - 1 > wp0 && j0 < wp0 + 31;
    };
    auto alibi_fix = [&](auto xb, int t) __attribute__((always_inline)) {
      constexpr int X = decltype(xb)::value;
      if (alibi_straddle(t)) {
        keep_branch();
        const float pl = alibi_pl(t);
#pragma unroll
        for (int e = 0; e < MB * 16; ++e) {
          const float jr = (float)(32 * (e / 16) + 8 * ((e % 16) >> 2) + (e % 4));
          sb[X][e / 16][e % 16] =
              __builtin_fmaf(__builtin_fabsf(pl - jr), -b2, sb[X][e / 16][e % 16] * c);
        }
      }
    };
    auto alibi_coef = [&](int t, float& cc, float& bb, float& ll) __attribute__((always_inline)) {
      const bool str = alibi_straddle(t);
      const bool right = !mk.causal && (t_begin + t) * BC >= wp0 + 31;   // every key >= every query
      cc = str ? 1.f : c;
      bb = str ? 0.f : right ? -b2 : b2;
      ll = __builtin_fmaf(-bb, alibi_pl(t), -alibi_base());
    };
    auto alibi_y = [&](auto xb, auto lo_c, auto hi_c, float cc, float bb, float ll)
                       __attribute__((always_inline)) {
      constexpr int X = decltype(xb)::value, LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
#pragma unroll
      for (int e = LO; e < HI; ++e) {
        const float jr = (float)(32 * (e / 16) + 8 * ((e % 16) >> 2) + (e % 4));
        sb[X][e / 16][e % 16] = __builtin_fmaf(sb[X][e / 16][e % 16], cc, __builtin_fmaf(bb, jr, ll));
      }
    };
    // ALIBI: the row statistics of y (relative to base): max, then the reference update with
    // m_tile = max + base
    auto update_ref_y = [&](float ext, float base) __attribute__((always_inline)) {
      ext = max_with_partner(ext);
      const float m_tile = ext + base;                  // -inf when no key of the tile shows
      const float g = m_tile - m_ref;                   // +huge on a row's first visible tile
      const float l_row = sum_with_partner(l_run);
      const bool heavy = exp2_fast(g + 4.f) > l_row;
      const bool move = (g > 0.f) & ((g > kTau) | heavy);
      m_prev = m_ref;
      m_ref = move ? m_tile : m_ref;
      moved = move;
    };
    // ALIBI: where a reference moved, y relative to the new one (the rare branch)
    auto alibi_rebase = [&](auto xb, float base) __attribute__((always_inline)) {
      constexpr int X = decltype(xb)::value;
      if (__any(moved)) {
        keep_branch();
        const float dm = m_ref - base;
#pragma unroll
        for (int e = 0; e < MB * 16; ++e) sb[X][e / 16][e % 16] -= dm;
      }
    };
    using Z = std::integral_constant<int, 0>;
    using NE = std::integral_constant<int, MB * 16>;
    auto alu0 = [&](auto xb) __attribute__((always_inline)) {
      float ext;
      if constexpr (ALIBI) {
        const float base = alibi_base();
        float cc, bb, ll;
        alibi_fix(xb, 0);
        alibi_coef(0, cc, bb, ll);
        alibi_y(xb, Z{}, NE{}, cc, bb, ll);
        row_max(xb, Z{}, NE{}, ext);
        update_ref_y(ext, base);
        alibi_rebase(xb, base);
      } else {
        row_max(xb, Z{}, NE{}, ext);
        update_ref(ext);
        shift(xb, Z{}, NE{});
      }
    };
    // ALU1 of S_Y, pair pp of its elements: P = 2^x (exp_pair), then l += P (fp32, in four
    // partial sums) and P rounded to the input type (sum_pair)
    auto exp_pair = [&](auto yb, auto ppc, float (&p)[2]) __attribute__((always_inline)) {
      constexpr int Y = decltype(yb)::value, pp = decltype(ppc)::value;
      constexpr int mb = pp / 8, r = 2 * (pp % 8);
      p[0] = exp2_fast(sb[Y][mb][r]);
      p[1] = exp2_fast(sb[Y][mb][r + 1]);
    };
    auto sum_pair = [&](auto ppc, const float (&p)[2], float (&part)[4]) __attribute__((always_inline)) {
      constexpr int pp = decltype(ppc)::value;
      constexpr int mb = pp / 8, r = 2 * (pp % 8), slot = pp & 3;
      if constexpr (pp < 4)
        part[slot] = p[0] + p[1];
      else
        part[slot] += p[0] + p[1];
      pk[mb][r >> 1] = pack2<BF16>(p[0], p[1]);
    };
    auto alu1 = [&](auto yb) __attribute__((always_inline)) {
      float part[4];
      static_for<MB * 8>([&](auto ppc) __attribute__((always_inline)) {
        float p[2];
        exp_pair(yb, ppc, p);
        sum_pair(ppc, p, part);
      });
      l_run += (part[0] + part[1]) + (part[2] + part[3]);
    };
    // O and l follow a moved reference (rare): alpha = 2^(m_old - m_new), 1 where the row's
    // reference stayed, 0 on a row's first visible tile
    auto rescale = [&]() __attribute__((always_inline)) {
      if (__any(moved)) {
        keep_branch();                  // not to be turned into multiplies by 1 on every tile
        const float alpha = exp2_fast(m_prev - m_ref);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      }
      moved = false;
    };

    // ---- phases.  Each MFMA is followed by its share of the phase's VALU work, and a
    // scheduling barrier keeps that order: the MFMA runs while the VALU work issues, and the
    // exponentials are spread evenly instead of being bunched.
    // GEMM0 + ALU1, and the V^T operand reads of ring stage stv spread over its MFMA slots
    auto compute_a = [&](auto xb, auto yb, auto stv) __attribute__((always_inline)) {
      constexpr int NP = (MB * 8) / (MB * KS);                                  // pairs per MFMA
      static_assert(NP * MB * KS == MB * 8, "pairs split evenly over the MFMAs");
      constexpr int NR = 2 * KK * DB, RPS = NR / (MB * KS);                     // reads per slot
      static_assert(RPS * MB * KS == NR, "reads split evenly over the MFMAs");
      // slot e: product e, the exponentials of its pairs, and the sums and conversions of the
      // previous slot's pairs (so that no instruction waits for an exponential just issued)
      float part[4], p[2][NP][2];
      static_for<MB * KS + 1>([&](auto ec) __attribute__((always_inline)) {
        constexpr int e = decltype(ec)::value;
        if constexpr (e < MB * KS) {
          qk(xb, ec);
          static_for<RPS>([&](auto rc) __attribute__((always_inline)) {
            read_v_one(stv, std::integral_constant<int, e * RPS + decltype(rc)::value>{});
          });
          static_for<NP>([&](auto pc) __attribute__((always_inline)) {
            constexpr int j = decltype(pc)::value;
            exp_pair(yb, std::integral_constant<int, e * NP + j>{}, p[e & 1][j]);
          });
        }
        if constexpr (e > 0) {
          static_for<NP>([&](auto pc) __attribute__((always_inline)) {
            constexpr int j = decltype(pc)::value;
            sum_pair(std::integral_constant<int, (e - 1) * NP + j>{}, p[(e - 1) & 1][j], part);
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      l_run += (part[0] + part[1]) + (part[2] + part[3]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 8; ++r) pin(pk[mb][r]);
      pin(l_run);
    };
    // GEMM1 + ALU0: the row max under the first MFMAs, the reference update under the next,
    // the shift spread over the rest
    // (with the K operand reads of ring stage stk spread over its MFMA slots)
    // (ALIBI: the ALU0 of key tile t is y first, over the first NT slots, then the row max and
    // the reference update; the move of y to a new reference follows the phase)
    auto compute_b = [&](auto xb, auto stk, int t) __attribute__((always_inline)) {
      constexpr int X = decltype(xb)::value;
      constexpr int NM = KK * DB, NX = 2;            // NX MFMA slots for the row max
      static_assert(NM >= 8, "ALU0 spread needs eight MFMA slots");
      constexpr int NR = MB * KS;                     // K reads, at most one per slot from slot 0
      static_assert(NR <= NM, "one K read per MFMA slot");
      constexpr int NT = 4;                           // ALIBI: slots for y
      float ext;
      float base = 0.f, cc = 0.f, bb = 0.f, ll = 0.f;
      if constexpr (ALIBI) {
        base = alibi_base();
        alibi_coef(t, cc, bb, ll);
      }
      static_for<NM>([&](auto ec) __attribute__((always_inline)) {
        constexpr int e = decltype(ec)::value;
        pv(ec);
        if constexpr (e < NR) read_k_one(stk, ec);
        if constexpr (ALIBI) {
          if constexpr (e < NT) {
            constexpr int LO = (NE::value * e) / NT, HI = (NE::value * (e + 1)) / NT;
            alibi_y(xb, std::integral_constant<int, LO>{}, std::integral_constant<int, HI>{}, cc, bb, ll);
          } else if constexpr (e < NT + NX) {
            constexpr int LO = (NE::value * (e - NT)) / NX, HI = (NE::value * (e - NT + 1)) / NX;
            row_max(xb, std::integral_constant<int, LO>{}, std::integral_constant<int, HI>{}, ext);
          } else if constexpr (e == NT + NX) {
            update_ref_y(ext, base);
          }
        } else if constexpr (e < NX) {
          constexpr int LO = (NE::value * e) / NX, HI = (NE::value * (e + 1)) / NX;
          row_max(xb, std::integral_constant<int, LO>{}, std::integral_constant<int, HI>{}, ext);
        } else if constexpr (e == NX) {
          update_ref(ext);
        } else {
          constexpr int J = e - NX - 1, NJ = NM - NX - 1;
          constexpr int LO = (NE::value * J) / NJ, HI = (NE::value * (J + 1)) / NJ;
          shift(xb, std::integral_constant<int, LO>{}, std::integral_constant<int, HI>{});
        }
        __builtin_amdgcn_sched_barrier(0);
      });
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) pin(sb[X][mb]);
      pin(l_run);
      pin(m_ref);
      pin(m_prev);
      if constexpr (ALIBI) alibi_rebase(xb, base);
    };
    // The scheduler would otherwise sink the operand reads below the phase's interleaved
    // MFMA/VALU groups, right in front of the wait for them, leaving their latency exposed.
    // K operands of the next tile stay in their registers until the read that fills them is
    // waited for, also where the next tile is never computed (the reads are untracked)
    auto keep_kop = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) keep(kop[mb][ks]);
    };
    auto issue_reads_now = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
    };
    // KPM: the padding word of tile t (LDS; read at the start of the step that masks it)
    auto pad_word = [&](int t) __attribute__((always_inline)) {
      if constexpr (KPM) return pwords[t + pw_off];
      else return 0ull;
    };
    // padding keys' scores -> -inf: element (mb, r) of a lane of half hi holds key
    // 32 mb + 8 (r / 4) + 4 hi + r % 4 of the tile
    auto pad_mask = [&](auto xb, unsigned long long pad) __attribute__((always_inline)) {
      constexpr int X = decltype(xb)::value;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        static_for<16>([&](auto rc) __attribute__((always_inline)) {
          constexpr int r = decltype(rc)::value;
          // bit k of the word (lanes 0-31) and bit k + 4 (lanes 32-63), each spread over a
          // half of the lane mask by an arithmetic shift
          const unsigned w = (unsigned)(pad >> (32 * mb));
          constexpr int k = 8 * (r >> 2) + (r & 3);
          const unsigned lo = (unsigned)((int)(w << (31 - k)) >> 31);
          const unsigned hi = (unsigned)((int)(w << (27 - k)) >> 31);
          const unsigned long long lanes = (unsigned long long)hi << 32 | lo;
          sb[X][mb][r] = __builtin_amdgcn_inverse_ballot_w64(lanes) ? NEG_INF : sb[X][mb][r];
        });
    };
    // (e: the entry of the tile; BLK: a tile this wave's query block does not select is hidden;
    // pw: KPM, the tile's padding word as read from LDS)
    auto mask_if_edge = [&](auto xb, int e, unsigned long long pw) __attribute__((always_inline)) {
      const bool hide = BLK && !entry_selected(e, stripe >> 1);
      unsigned long long pad = 0;
      if constexpr (KPM) {
        // (readfirstlane returns an int: each half goes through unsigned, not sign-extended)
        pad = (unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)pw) |
              (unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)(pw >> 32)) << 32;
      }
      const bool ed = edge(rel(e));
      if (hide || ed || pad != 0) {
        if (hide || ed) mask(xb, rel(e), hide);
        if constexpr (KPM) pad_mask(xb, pad);
      }
    };

    // Iteration i, ring stage U = i mod kNS; buffer (i+1) mod 2 receives S_{i+1}, buffer i mod 2
    // holds S_i.  Copies: each wave issues its chunks of K_{i+kPD+1} (stage U) and V_{i+kPD}
    // (stage U-1) at the start of iteration i; at the end of phase 1 it waits until only the
    // current iteration's copies are outstanding, and the barrier that ends the iteration
    // publishes everything older.  Tile t is first read in iteration t-2 (K) or t (V), after
    // that barrier of iteration t-3 or earlier; a stage is rewritten only in the iteration
    // after the barrier that follows the last read of its previous tile (iteration t-2 for K,
    // t for V).  The phase-1 fence covers the V^T reads of phase 1, the end-of-iteration wait
    // the K reads of phase 2.
    auto iteration = [&](auto uc, int i) __attribute__((always_inline)) {
      constexpr int U = decltype(uc)::value;
      using XB = std::integral_constant<int, (U + 1) & 1>;
      using YB = std::integral_constant<int, U & 1>;
      static_assert(kPD == 3, "entries of steps i + 1 .. i + 3 carried, i + 4 read ahead");
      int e1 = i + 1, ek = i + kPD + 1, ev = i + kPD;
      const unsigned long long pw1 = pad_word(i + 1);   // (KPM: the oldest LDS read of the step)
      if constexpr (BLK) {
        e1 = h1;
        ev = h3;
        ek = __builtin_amdgcn_readfirstlane(pre);
        pre = tlist[i + kPD + 2];         // the oldest LDS operation of the step
        h1 = h2;
        h2 = h3;
        h3 = ek;
      }
      issue_copies(ek, ev, U, (U + kNS - 1) % kNS);
      issue_reads_now();
      compute_a(XB{}, YB{}, std::integral_constant<int, U>{});   // GEMM0_{i+1} + ALU1_i, V_i reads
      wait_vmcnt<2 * CPT * (kPD - 2)>();
      wait_lgkmcnt0_fence();             // V_i operands have landed (GEMM1_i stays below)
      mask_if_edge(XB{}, e1, pw1);
      if constexpr (ALIBI) alibi_fix(XB{}, i + 1);
      compute_b(XB{}, std::integral_constant<int, (U + 2) % kNS>{}, i + 1);   // GEMM1_i + ALU0_{i+1}, K_{i+2} reads
      rescale();
      wait_lgkmcnt0();
      keep_kop();                        // no register of an in-flight read is reused before the wait
      wg_barrier();
    };
    // first iteration (i = -1): only S_0 and its row statistics
    auto iteration_first = [&]() __attribute__((always_inline)) {
      using X = std::integral_constant<int, 0>;
      const int e0 = ent(0);
      const unsigned long long pw0 = pad_word(0);
      issue_copies(ent(kPD), ent(kPD - 1), kPD % kNS, (kPD - 1) % kNS);
      static_for<MB * KS>([&](auto ec) __attribute__((always_inline)) { qk(X{}, ec); });
      wait_vmcnt<2 * CPT * (kPD - 2)>();
      mask_if_edge(X{}, e0, pw0);
      read_k(std::integral_constant<int, 1>{});
      issue_reads_now();
      alu0(X{});
      rescale();
      wait_lgkmcnt0();
      wg_barrier();
    };
    // last iteration (i = T-1, ring stage U): only P_{T-1} and its product with V_{T-1}
    auto iteration_last = [&](auto uc) __attribute__((always_inline)) {
      constexpr int U = decltype(uc)::value;
      using YB = std::integral_constant<int, U & 1>;
      // beyond the sequence: zero fills, uniform vmcnt
      issue_copies(BLK ? 0xffff : T + kPD, BLK ? 0xffff : T + kPD - 1, U, (U + kNS - 1) % kNS);
      read_v(std::integral_constant<int, U>{});
      issue_reads_now();
      alu1(YB{});
      wait_vmcnt<2 * CPT * (kPD - 2)>();
      wait_lgkmcnt0_fence();
      static_for<KK * DB>([&](auto ec) __attribute__((always_inline)) { pv(ec); });
      wg_barrier();
    };

    // ---- prologue: copies of K_0..K_{kPD-1} and V_0..V_{kPD-2}, all waited for
#pragma unroll
    for (int t = 0; t < kPD - 1; ++t) {
      const int e = ent(t);
      issue_copies(e, e, t % kNS, t % kNS);
    }
    {
      const int tk = rel(ent(kPD - 1));
      const int ok = tk < T ? (t_begin + tk) * TILE : head_bytes;
#pragma unroll
      for (int j = 0; j < CPT; ++j)
        buffer_load16_lds(rk, kring + ((kPD - 1) % kNS) * TILE + 16 * kThreads * j + 1024 * wave,
                          cp_src + 16 * kThreads * j + ok);
    }
    wait_vmcnt<0>();
    wg_barrier();
    read_k(std::integral_constant<int, 0>{});
    wait_lgkmcnt0_fence();

    using U0 = std::integral_constant<int, 0>;
    using U1 = std::integral_constant<int, 1>;
    using U2 = std::integral_constant<int, 2>;
    using U3 = std::integral_constant<int, 3>;
    static_assert(kNS == 4, "the loop is unrolled over four ring stages");
    iteration_first();
    int i = 0;
    for (; i + kNS <= TT - 1; i += kNS) {
      iteration(U0{}, i);
      iteration(U1{}, i + 1);
      iteration(U2{}, i + 2);
      iteration(U3{}, i + 3);
    }
    const int rem = TT - 1 - i;        // 0 .. kNS-1 iterations left, then the last
    if (rem > 0) iteration(U0{}, i);
    if (rem > 1) iteration(U1{}, i + 1);
    if (rem > 2) iteration(U2{}, i + 2);
    if (rem == 0)
      iteration_last(U0{});
    else if (rem == 1)
      iteration_last(U1{});
    else if (rem == 2)
      iteration_last(U2{});
    else
      iteration_last(U3{});
    wait_vmcnt<0>();                   // no copy may land after this tile is done

    // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l)
    const float l_tot = sum_with_partner(l_run);
    if (qi < n) {
      // a row that saw no key (fewer keys than queries, or a window past every key): O = 0
      const bool live = l_tot > 0.f;
      const float inv = live ? 1.f / l_tot : 0.f;
      char* orow = a.o + head + (long)qi * RB;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int dim = 32 * db + 8 * gq + 4 * hi;
          u32x2 w = {pack2<BF16>(oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv),
                     pack2<BF16>(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + dim * 2) = w;
        }
      if (a.lse != nullptr && hi == 0)
        a.lse[lrow + qi] = live ? (m_ref + __builtin_log2f(l_tot)) * kLn2 : NEG_INF;
    } else if (PADDED && qi < nw) {   // a padding row
      char* orow = a.o + head + (long)qi * RB;
#pragma unroll
      for (int c16 = 0; c16 < RB / 32; ++c16)
        *reinterpret_cast<u32x4*>(orow + 32 * c16 + 16 * hi) = u32x4{};
      if (a.lse != nullptr && hi == 0) a.lse[lrow + qi] = NEG_INF;
    }
  }
}

// nq query rows over nk key rows (dense [B, H, rows, D] operands), query i at key position
// i + nk - nq; nq == nk for self-attention and padded batches
// slopes: ALiBi slopes [H] (device) or null
template <int D, bool BF16>
hipError_t launch(const FwdParams& p, int nq, int nk, hipStream_t stream,
                  const float* slopes = nullptr, const unsigned char* blocks = nullptr,
                  const unsigned char* kpm = nullptr) {
  MainArgs a;
  a.q = static_cast<const char*>(p.q);
  a.k = static_cast<const char*>(p.k);
  a.v = static_cast<const char*>(p.v);
  a.o = static_cast<char*>(p.o);
  a.lse = p.lse;
  a.seqlens = p.seqlens;
  a.cu = p.cu;
  a.total = p.total;
  a.n = nq;
  a.nk = nk;
  a.off = nk - nq;
  a.heads = p.H;
  a.n_bh = p.B * p.H;
  a.n_qt = (nq + kBr - 1) / kBr;
  // Pairing balances causal rows whose visible key count grows with the query index.  With the
  // queries at the end of a longer key sequence (a.off > 0) that count hardly changes: tile t
  // sees about off + 128 t keys, so the last tile does less than twice the first's work unless
  // nq >= off + 256.  There pairing would gain nothing and would put twice as many heads in
  // flight on an XCD, whose K/V then outgrow its L2.
  const bool growing = p.causal && p.window_left < 0 && nq >= a.off + 2 * kBr;
  a.paired = growing && (long)a.n_bh * ((a.n_qt + 1) / 2) >= 256;
  a.n_units = a.paired ? (a.n_qt + 1) / 2 : a.n_qt;
  // a zero scale becomes a tiny one: every probability is then exactly 1 (as for 0) while
  // hidden scores (-inf) still give 0 instead of -inf * 0 = NaN
  a.c = (float)(std::fmax(std::fabs((double)p.scale), 1e-30) * 1.4426950408889634);
  a.q_sign = p.scale < 0.f ? 0x80008000u : 0u;
  a.causal = p.causal;
  a.wl = p.window_left;
  a.wr = p.causal ? 0 : p.window_right;
  a.slopes = slopes;
  a.blocks = blocks;
  a.kpm = kpm;
  a.n_qb = (nq + 63) / 64;
  a.n_kb = (nk + 63) / 64;
  const long wgs = (long)a.n_bh * a.n_units;
  if (slopes != nullptr)   // (no padded batch takes ALiBi or a block mask)
    hipLaunchKernelGGL((fwd_main_kernel<D, BF16, false, true>), dim3((unsigned)wgs),
                       dim3(kThreads), 0, stream, a);
  else if (blocks != nullptr)
    hipLaunchKernelGGL((fwd_main_kernel<D, BF16, false, false, true>), dim3((unsigned)wgs),
                       dim3(kThreads), 0, stream, a);
  else if (kpm != nullptr)
    hipLaunchKernelGGL((fwd_main_kernel<D, BF16, false, false, false, true>), dim3((unsigned)wgs),
                       dim3(kThreads), 0, stream, a);
  else if (p.seqlens != nullptr || p.cu != nullptr)
    hipLaunchKernelGGL((fwd_main_kernel<D, BF16, true>), dim3((unsigned)wgs), dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((fwd_main_kernel<D, BF16, false>), dim3((unsigned)wgs), dim3(kThreads),
                       0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_main(const FwdParams& p, hipStream_t stream) {
  if (p.D == 64) return p.bf16 ? launch<64, true>(p, p.N, p.N, stream) : launch<64, false>(p, p.N, p.N, stream);
  return p.bf16 ? launch<128, true>(p, p.N, p.N, stream) : launch<128, false>(p, p.N, p.N, stream);
}

bool fwd_main_takes_blocks(int D, int nk) {
  const int bc = D == 64 ? Shape<64>::BC : Shape<128>::BC;
  return (nk + bc - 1) / bc <= kListMax;
}

hipError_t launch_fwd_main_kv(const KvParams& p, hipStream_t stream) {
  FwdParams f;
  f.q = p.q;
  f.k = p.k;
  f.v = p.v;
  f.o = p.o;
  f.lse = p.lse;
  f.seqlens = nullptr;
  f.cu = nullptr;
  f.B = p.B;
  f.H = p.H;
  f.N = p.Nq;
  f.D = p.D;
  f.bf16 = p.bf16;
  f.scale = p.scale;
  f.causal = p.causal;
  f.window_left = p.window_left;
  f.window_right = p.window_right;
  if ((p.blocks != nullptr || p.kpm != nullptr) && !fwd_main_takes_blocks(p.D, p.Nk))
    return hipErrorInvalidValue;   // more key tiles than a tile list holds
  if (p.D == 64)
    return p.bf16 ? launch<64, true>(f, p.Nq, p.Nk, stream, p.slopes, p.blocks, p.kpm)
                  : launch<64, false>(f, p.Nq, p.Nk, stream, p.slopes, p.blocks, p.kpm);
  return p.bf16 ? launch<128, true>(f, p.Nq, p.Nk, stream, p.slopes, p.blocks, p.kpm)
                : launch<128, false>(f, p.Nq, p.Nk, stream, p.slopes, p.blocks, p.kpm);
}

}  // namespace fa
