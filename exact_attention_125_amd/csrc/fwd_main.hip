// Fused attention forward for gfx950: the kernel for grids that fill the chip.
//
// A workgroup of 8 waves owns tiles of 256 query rows of one (batch, head), 32 rows per
// wave.  The key/value sequence is processed in tiles of BC keys (64 for head dim 64, 32
// for 128).  Per key tile j each wave does
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
//   phase 1  V_j operands LDS -> registers (issued first, land under the compute);
//            GEMM0_{j+1} interleaved with ALU1_j
//   phase 2  edge mask of S_{j+1}; K_{j+2} operands LDS -> registers;
//            GEMM1_j interleaved with ALU0_{j+1}; O rescaled where a reference moved
//
// sched_group_barrier interleaves each phase's MFMAs with its VALU work, and empty asm
// statements keep each phase's VALU results from being sunk into the next phase.  K and V
// tiles arrive by direct global->LDS copies (no registers, no LDS write instructions) into
// rings of kNS stages, issued kPD tiles ahead; the 16-byte chunks are placed so that the
// LDS layout is the XOR-swizzled one the operand reads expect (no bank conflicts).  One
// workgroup barrier per key tile publishes the copies and guards ring reuse.
//
// Under a causal mask with no left window bound the work of a query tile grows with its
// index; there a workgroup processes two query tiles, qt and n_qt - 1 - qt, so that every
// workgroup has the same amount of work (when that still leaves a workgroup per CU).  Every wave computes every key tile the
// workgroup visits; tiles hidden from some or all of a wave's queries go through the mask
// and contribute P = 0.
//
// The arithmetic follows the tiling of "告别OOM和训练慢：用Flash Attention加速你的PyTorch大模型
// （含A100环境配置）" §2.1 with the running max / running sum of its §2.2 (read as
// l_new = exp(m_old - m_new) l_old + sum exp(s - m_new), O rescaled by the same factor and
// divided by l once at the end), one query block against all visible key blocks as "Flash
// Attention 3.7 核心原理与实战：加速Transformer模型训练与推理" §3.1 describes.  The reference m of a
// row is the exact maximum of its first visible tile and moves to a later tile's exact
// maximum when that one is not negligible against the mass already summed (2^g * 16 > l) or
// exceeds m by more than 2^kTau; the softmax does not depend on the shift (the safe-softmax
// argument of the same §2.2), rows dominated by a few keys keep a largest probability of
// exactly 1, and probabilities stay below 2^kTau.  l is summed in fp32 from unrounded
// probabilities; P is rounded once to the input type; LSE = ln 2 * (m + log2 l).
#include <cmath>
#include <type_traits>

#include "cdna4.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kThreads = 512;      // 8 waves
constexpr int kBr = 256;           // query rows per query tile (32 per wave)
constexpr int kPD = 4;             // key tiles copied ahead
constexpr int kNS = kPD + 1;       // LDS ring stages, K and V each
constexpr float kTau = 8.0f;
constexpr float kNoRef = -1e30f;   // reference of a row with no visible key yet

struct MainArgs {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int n;          // sequence length
  int n_bh;       // batch * heads
  int n_qt;       // query tiles per head
  int n_units;    // workgroups per head: n_qt, or ceil(n_qt / 2) query-tile pairs
  int paired;     // a workgroup takes query tiles u and n_qt - 1 - u
  float c;        // max(|softmax_scale|, tiny) * log2(e)
  unsigned q_sign;  // 0x80008000 negates Q (negative scale)
  int causal, wl, wr;
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
  static_assert(TILE == 16 * kThreads, "one 16-byte chunk per thread per tile");
  static_assert(kPD >= 2, "the phase-1 wait keeps one iteration of copies in flight");
};

template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void fwd_main_kernel(MainArgs a) {
  using S = Shape<D>;
  constexpr int BC = S::BC, MB = S::MB, KS = S::KS, DB = S::DB, KK = S::KK, RB = S::RB;

  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * kNS * S::TILE];
  char FA_LDS* kring = (char FA_LDS*)lds_raw;
  char FA_LDS* vring = kring + kNS * S::TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, unit;
  xcd_tile_order(blockIdx.x, a.n_bh, a.n_units, bh, unit);
  const int n = a.n;
  const long head = (long)bh * n * RB;
  const int head_bytes = n * RB;
  const auto rq = make_rsrc(a.q + head, head_bytes);
  const auto rk = make_rsrc(a.k + head, head_bytes);
  const auto rv = make_rsrc(a.v + head, head_bytes);
  const Mask mk{n, a.causal, a.wl, a.wr};
  const float c = a.c;
  const float NEG_INF = -__builtin_inff();

  // The two waves of a SIMD (w and w + 4) own neighbouring 32-row stripes, so under a
  // causal mask they have nearly the same number of visible keys.
  const int stripe = 2 * (wave & 3) + (wave >> 2);

  // ---- per-lane constants
  // transposing-read coordinates (see cdna4.h): 16-lane group, row, quad
  const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
  const int tr_key = (tg >> 1) * 4 + tr;
  const int tr_byte = (tq & 1) * 8;
  // LDS offsets inside a stage, independent of the stage: K operand of k-step ks (row l32,
  // chunk 2 ks + hi; the 32-key block mb adds 32 rows) and V^T operand halves h (rows
  // tr_key + 8 h) of dim block db (the 16-key step kk adds 16 rows).  The swizzle of a row
  // depends only on bits that adding 32 or 16 rows leaves alone.
  int kb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kb[ks] = tile_offset<D>(l32, 2 * ks + hi);
  unsigned vb[2][DB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      vb[h][db] = tile_offset<D>(tr_key + 8 * h, 4 * db + 2 * (tg & 1) + (tq >> 1)) + tr_byte;
  // async copies: thread tid fills physical 16-byte chunk tid of each tile
  const int cp_row = (16 * tid) / RB;
  const int cp_src = cp_row * RB + ((((16 * tid) % RB) / 16) ^ chunk_swizzle<D>(cp_row)) * 16;

  const int npass = (a.paired && a.n_qt - 1 - unit != unit) ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
    const int qt = a.paired ? (pass == 0 ? a.n_qt - 1 - unit : unit) : unit;
    if (pass > 0) wg_barrier();      // the previous tile's last LDS reads are done

    const int q0 = qt * kBr;
    const int wq0 = q0 + 32 * stripe;
    const int qi = wq0 + l32;

    i16x8 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = buffer_load16(rq, qi * RB + (2 * ks + hi) * 16);
      x ^= a.q_sign;
      qreg[ks] = __builtin_bit_cast(i16x8, x);
    }

    int key_lo, key_hi;
    mk.key_range(q0, min(q0 + kBr - 1, n - 1), key_lo, key_hi);
    const int t_begin = key_lo / BC;
    const int T = (key_hi + BC - 1) / BC - t_begin;   // key tiles the workgroup visits (>= 1)
    // visible key interval of this lane's query (edge tiles)
    const int row_lo = mk.wl >= 0 ? max(0, qi - mk.wl) : 0;
    const int row_hi = min(n - 1, mk.causal ? qi : (mk.wr >= 0 ? qi + mk.wr : n - 1));

    auto issue_copies = [&](int tk, int tv) __attribute__((always_inline)) {
      // tiles past the last one read beyond the buffer: zero fills, no memory traffic
      const int ok = tk < T ? (t_begin + tk) * BC * RB : head_bytes;
      const int ov = tv < T ? (t_begin + tv) * BC * RB : head_bytes;
      buffer_load16_lds(rk, kring + (tk % kNS) * S::TILE + 1024 * wave, cp_src + ok);
      buffer_load16_lds(rv, vring + (tv % kNS) * S::TILE + 1024 * wave, cp_src + ov);
    };

    // ---- per-wave state of this query tile
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m_ref = kNoRef, l_run = 0.f, alpha = 1.f;
    bool moved = false;
    f32x16 sb[2][MB];
    unsigned pk[MB][8];
    i16x8 kop[MB][KS];
    // V^T operands as the two halves the transposing reads return, joined where the MFMA
    // uses them (after the wait), so no copy of them can run before the data has landed
    i16x4 vlo[KK][DB], vhi[KK][DB];

    auto edge = [&](int t) __attribute__((always_inline)) {
      const int j0 = (t_begin + t) * BC;
      return !mk.all_visible(wq0, wq0 + 31, j0, j0 + BC);
    };

    // ---- the pieces of work
    auto read_k = [&](int t) __attribute__((always_inline)) {
      const char FA_LDS* kt = kring + (t % kNS) * S::TILE;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          kop[mb][ks] = __builtin_bit_cast(i16x8, lds_read16(kt + kb[ks], 32 * mb * RB));
    };
    // V^T operands, read without compiler-inserted waits (see lds_read_tr_nowait); they are
    // used only after a wait_lgkmcnt0.
    auto read_v = [&](int t) __attribute__((always_inline)) {
      const unsigned base = lds_addr(vring) + (t % kNS) * S::TILE;
      unsigned va[2][DB];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < DB; ++db) va[h][db] = base + vb[h][db];
      static_for<KK>([&](auto kkc) __attribute__((always_inline)) {
        constexpr int kk = decltype(kkc)::value;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          vlo[kk][db] = lds_read_tr_nowait<kk * 16 * RB>(va[0][db]);
          vhi[kk][db] = lds_read_tr_nowait<kk * 16 * RB>(va[1][db]);
        }
      });
    };
    auto gemm0 = [&](auto xb) __attribute__((always_inline)) {
      constexpr int X = decltype(xb)::value;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) sb[X][mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          sb[X][mb] = mfma32x32x16<BF16>(kop[mb][ks], qreg[ks], sb[X][mb]);
    };
    auto gemm1 = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 pb = {pk[kk >> 1][4 * (kk & 1) + 0], pk[kk >> 1][4 * (kk & 1) + 1],
                          pk[kk >> 1][4 * (kk & 1) + 2], pk[kk >> 1][4 * (kk & 1) + 3]};
#pragma unroll
        for (int db = 0; db < DB; ++db)
          oacc[db] = mfma32x32x16<BF16>(__builtin_shufflevector(vlo[kk][db], vhi[kk][db], 0, 1, 2, 3, 4, 5, 6, 7),
                                        __builtin_bit_cast(i16x8, pb), oacc[db]);
      }
    };
    // hidden scores -> -inf (edge tiles only)
    auto mask = [&](auto xb, int t) __attribute__((always_inline)) {
      constexpr int X = decltype(xb)::value;
      const int base = (t_begin + t) * BC + 4 * hi;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = base + 32 * mb + 8 * (r >> 2) + (r & 3);
          sb[X][mb][r] = (j >= row_lo && j <= row_hi) ? sb[X][mb][r] : NEG_INF;
        }
    };
    // row max, reference update, x = s*c - m (in place)
    auto alu0 = [&](auto xb) __attribute__((always_inline)) {
      constexpr int X = decltype(xb)::value;
      float ext = sb[X][0][0];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = (mb == 0 ? 1 : 0); r < 16; ++r) ext = fmaxf(ext, sb[X][mb][r]);
      ext = max_with_partner(ext);
      const float m_tile = ext * c;                     // -inf when no key of the tile shows
      const float g = m_tile - m_ref;                   // +huge on a row's first visible tile
      const float l_row = sum_with_partner(l_run);      // both lanes of a row decide alike
      const bool heavy = exp2_fast(g + 4.f) > l_row;
      const bool move = (g > 0.f) & ((g > kTau) | heavy);
      alpha = move ? exp2_fast(m_ref - m_tile) : 1.f;   // 0 on a row's first visible tile
      l_run *= alpha;
      m_ref = move ? m_tile : m_ref;
      moved = move;
      const float neg_m = -m_ref;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sb[X][mb][r] = __builtin_fmaf(sb[X][mb][r], c, neg_m);
    };
    // P = 2^x, l += P (fp32), P rounded to the input type
    auto alu1 = [&](auto yb) __attribute__((always_inline)) {
      constexpr int Y = decltype(yb)::value;
      float part[4];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = exp2_fast(sb[Y][mb][r]);
          const float p1 = exp2_fast(sb[Y][mb][r + 1]);
          const int slot = (r >> 1) & 3;
          part[slot] = (mb == 0 && r < 8) ? p0 + p1 : part[slot] + (p0 + p1);
          pk[mb][r >> 1] = pack2<BF16>(p0, p1);
        }
      l_run += (part[0] + part[1]) + (part[2] + part[3]);
    };
    auto rescale = [&]() __attribute__((always_inline)) {
      if (__any(moved)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      }
      moved = false;
    };

    // ---- phases
    auto compute_a = [&](auto xb, auto yb) __attribute__((always_inline)) {   // GEMM0 + ALU1
      gemm0(xb);
      alu1(yb);
#pragma unroll
      for (int e = 0; e < MB * KS; ++e) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, (MB * 40) / (MB * KS), 0);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 8; ++r) pin(pk[mb][r]);
      pin(l_run);
    };
    auto compute_b = [&](auto xb) __attribute__((always_inline)) {            // GEMM1 + ALU0
      gemm1();
      alu0(xb);
#pragma unroll
      for (int e = 0; e < KK * DB; ++e) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, (MB * 32 + 16) / (KK * DB), 0);
      }
      constexpr int X = decltype(xb)::value;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) pin(sb[X][mb]);
      pin(l_run);
      pin(m_ref);
      pin(alpha);
    };
    auto mask_if_edge = [&](auto xb, int t) __attribute__((always_inline)) {
      if (edge(t)) mask(xb, t);
    };

    // Iteration i; X holds S_{i+1}, Y holds S_i.  Copies: each wave issues its chunk of
    // K_{i+kPD+1} and V_{i+kPD} at the start of iteration i into ring stage (tile % kNS); at
    // the end of phase 1 it waits until only the current iteration's copies are
    // outstanding, and the barrier that ends the iteration publishes everything older.
    // Tile t is first read in iteration t-2 (K) or t (V), after that barrier of iteration
    // t-3 or earlier; a stage is rewritten only in the iteration after the barrier that
    // follows the last read of its previous tile (iteration t-2 for K, t for V).
    auto iteration = [&](auto xb, auto yb, int i) __attribute__((always_inline)) {
      issue_copies(i + kPD + 1, i + kPD);
      read_v(i);
      compute_a(xb, yb);                 // GEMM0_{i+1} + ALU1_i
      wait_vmcnt<2 * (kPD - 2)>();
      wait_lgkmcnt0_fence();             // V_i operands have landed (GEMM1_i stays below)
      mask_if_edge(xb, i + 1);
      read_k(i + 2);
      compute_b(xb);                     // GEMM1_i + ALU0_{i+1}
      rescale();
      wait_lgkmcnt0();
      wg_barrier();
    };
    // first iteration (i = -1): only S_0 and its row statistics
    auto iteration_first = [&]() __attribute__((always_inline)) {
      using X = std::integral_constant<int, 0>;
      issue_copies(kPD, kPD - 1);
      gemm0(X{});
      wait_vmcnt<2 * (kPD - 2)>();
      mask_if_edge(X{}, 0);
      read_k(1);
      alu0(X{});
      rescale();
      wait_lgkmcnt0();
      wg_barrier();
    };
    // last iteration (i = T-1): only P_{T-1} and its product with V_{T-1}
    auto iteration_last = [&](auto yb) __attribute__((always_inline)) {
      issue_copies(T + kPD, T + kPD - 1);   // beyond the sequence: zero fills, uniform vmcnt
      read_v(T - 1);
      alu1(yb);
      wait_vmcnt<2 * (kPD - 2)>();
      wait_lgkmcnt0_fence();
      gemm1();
      wg_barrier();
    };

    // ---- prologue: copies of K_0..K_{kPD-1} and V_0..V_{kPD-2}, all waited for
#pragma unroll
    for (int t = 0; t < kPD - 1; ++t) issue_copies(t, t);
    {
      const int tk = kPD - 1;
      const int ok = tk < T ? (t_begin + tk) * BC * RB : head_bytes;
      buffer_load16_lds(rk, kring + (tk % kNS) * S::TILE + 1024 * wave, cp_src + ok);
    }
    wait_vmcnt<0>();
    wg_barrier();
    read_k(0);

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    iteration_first();
    int i = 0;
    for (; i + 2 <= T - 1; i += 2) {
      iteration(I1{}, I0{}, i);        // i even: S_{i+1} -> buffer 1
      iteration(I0{}, I1{}, i + 1);    // i+1 odd: S_{i+2} -> buffer 0
    }
    if (i < T - 1) {
      iteration(I1{}, I0{}, i);
      ++i;
    }
    if (i & 1)
      iteration_last(I1{});
    else
      iteration_last(I0{});
    wait_vmcnt<0>();                   // no copy may land after this tile is done

    // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l)
    const float l_tot = sum_with_partner(l_run);
    if (qi < n) {
      const float inv = 1.f / l_tot;
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
        a.lse[(long)bh * n + qi] = (m_ref + __builtin_log2f(l_tot)) * kLn2;
    }
  }
}

template <int D, bool BF16>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  MainArgs a;
  a.q = static_cast<const char*>(p.q);
  a.k = static_cast<const char*>(p.k);
  a.v = static_cast<const char*>(p.v);
  a.o = static_cast<char*>(p.o);
  a.lse = p.lse;
  a.n = p.N;
  a.n_bh = p.B * p.H;
  a.n_qt = (p.N + kBr - 1) / kBr;
  // pairing balances causal rows whose visible key count grows with the query index
  const bool growing = p.causal && p.window_left < 0;
  a.paired = growing && (long)a.n_bh * ((a.n_qt + 1) / 2) >= 256;
  a.n_units = a.paired ? (a.n_qt + 1) / 2 : a.n_qt;
  // a zero scale becomes a tiny one: every probability is then exactly 1 (as for 0) while
  // hidden scores (-inf) still give 0 instead of -inf * 0 = NaN
  a.c = (float)(std::fmax(std::fabs((double)p.scale), 1e-30) * 1.4426950408889634);
  a.q_sign = p.scale < 0.f ? 0x80008000u : 0u;
  a.causal = p.causal;
  a.wl = p.window_left;
  a.wr = p.causal ? 0 : p.window_right;
  const long blocks = (long)a.n_bh * a.n_units;
  hipLaunchKernelGGL((fwd_main_kernel<D, BF16>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_main(const FwdParams& p, hipStream_t stream) {
  if (p.D == 64) return p.bf16 ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return p.bf16 ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace fa
