// Fused attention forward for grids too small to fill the chip: the keys of a query tile are
// split over the waves of one workgroup, and the partial results merge in LDS.
//
// A workgroup owns 64 query rows of one (batch, head) (two stripes of 32) and splits the key
// tiles those rows can see into KSPLIT contiguous parts (4 at head dim 64, 2 at 128); wave w
// takes stripe w % 2 of part w / 2.  The two waves of a part share its key / value tiles: 64
// keys per tile, double-buffered in LDS (global loads into registers, written to the other
// buffer while the current tile is computed).  Per tile each wave computes, as the four-wave
// kernel does,
//
//   S^T = K Q^T      32x32x16 MFMAs, Q^T in registers
//   mask             on tiles that straddle a causal / window / sequence edge
//   online softmax   a reference m per query (base 2), P = 2^(s c - m), l += P in fp32, P
//                    rounded once to the input type
//   O^T += V^T P^T   V^T from transposing LDS reads, P^T straight from the S^T registers
//
// and at the end the parts of a stripe merge by the log-sum-exp rule: each wave leaves its
// normalised partial O (fp32) and its LSE in LDS, and the wave of part 0 forms
// LSE = log2 sum_p 2^LSE_p, O = sum_p 2^(LSE_p - LSE) O_p.  The result is the attention of
// the whole row (the running max / running sum of "告别OOM和训练慢：用Flash Attention加速你的
// PyTorch大模型（含A100环境配置）" §2.2 applied once more, across the parts), with one rounding of
// O at the end.  A grid of B H N / 64 workgroups of 2 KSPLIT waves gives a small problem
// (B H N / 128 main-kernel workgroups, under one per CU) KSPLIT / 2 times the waves, each
// with a KSPLIT-th of the key loop.
#include <cmath>
#include <type_traits>

#include "cdna4.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kBqS = 64;          // query rows per workgroup
constexpr int kBcS = 64;          // keys per tile
constexpr float kTauS = 8.0f;     // largest lag (base 2) of the reference behind a row max

struct SplitArgs {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int n;          // rows per (batch, head)
  int n_bh;
  int n_qt;       // 64-row query tiles per head
  float c;        // max(|softmax_scale|, tiny) * log2(e)
  unsigned q_sign;
  int causal, wl, wr;
};

template <int D>
struct SplitShape {
  static constexpr int KSPLIT = D == 64 ? 4 : 2;        // key parts
  static constexpr int WAVES = 2 * KSPLIT;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int RB = 2 * D;                       // bytes per row
  static constexpr int TILE = kBcS * RB;                 // bytes per K or V tile
  static constexpr int LOADS = TILE / (16 * 128);        // 16-byte chunks per thread (2 waves)
  static constexpr int PART_LDS = 2 * 2 * TILE;          // two stages of K and V
  static constexpr int KS = D / 16, DB = D / 32;
  static_assert(LOADS * 16 * 128 == TILE, "whole chunks per thread");
  static_assert(KSPLIT * PART_LDS <= 160 * 1024, "LDS");
  // merge area: every wave's normalised O^T (D x 32 fp32) and LSE (32), per lane
  static_assert(WAVES * (D * 32 + 64) * 4 <= KSPLIT * PART_LDS, "merge area fits the rings");
};

template <int D, bool BF16>
__global__ __launch_bounds__(SplitShape<D>::THREADS, 1) void fwd_split_kernel(SplitArgs a) {
  using S = SplitShape<D>;
  constexpr int KSPLIT = S::KSPLIT, RB = S::RB, TILE = S::TILE, LOADS = S::LOADS, KS = S::KS,
                DB = S::DB, CPR = D / 8;

  __shared__ __attribute__((aligned(16))) char lds_raw[KSPLIT * S::PART_LDS];
  char FA_LDS* lds = (char FA_LDS*)lds_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int stripe = wave & 1, part = wave >> 1;
  const int ptid = tid & 127;   // thread index within the part's two waves

  int bh, qt;
  xcd_tile_order(blockIdx.x, a.n_bh, a.n_qt, bh, qt);
  const int n = a.n;
  const long head = (long)bh * n * RB;
  const auto rq = make_rsrc(a.q + head, n * RB);
  const auto rk = make_rsrc(a.k + head, n * RB);
  const auto rv = make_rsrc(a.v + head, n * RB);
  const Mask mk{n, a.causal, a.wl, a.wr};
  const float c = a.c;
  const float NEG_INF = -__builtin_inff();

  const int q0 = qt * kBqS;
  const int wq0 = q0 + 32 * stripe, wq1 = wq0 + 31;
  const int qi = wq0 + l32;

  i16x8 qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = buffer_load16(rq, qi * RB + (2 * ks + hi) * 16);
    x ^= a.q_sign;
    qreg[ks] = __builtin_bit_cast(i16x8, x);
  }

  // key tiles of the workgroup's rows, split into KSPLIT contiguous parts (the first ones one
  // tile longer when they do not divide evenly)
  int key_lo, key_hi;
  mk.key_range(q0, min(q0 + kBqS - 1, n - 1), key_lo, key_hi);
  const int t_lo = max(key_lo, 0) / kBcS;
  const int t_hi = max((max(key_hi, 0) + kBcS - 1) / kBcS, t_lo);
  const int nt = t_hi - t_lo, per = nt / KSPLIT, extra = nt % KSPLIT;
  const int p_begin = t_lo + part * per + min(part, extra);
  const int p_tiles = per + (part < extra ? 1 : 0);
  const int max_tiles = per + (extra > 0 ? 1 : 0);      // iterations of every wave
  int wkey_lo, wkey_hi;
  mk.key_range(wq0, min(wq1, n - 1), wkey_lo, wkey_hi);
  const bool wave_has_rows = wq0 < n;

  char FA_LDS* ring = lds + part * S::PART_LDS;
  u32x4 kbuf[LOADS], vbuf[LOADS];
  auto load_tile = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int cidx = ptid + 128 * i;
      const int row = t * kBcS + cidx / CPR, col = (cidx % CPR) * 16;
      kbuf[i] = buffer_load16(rk, row * RB + col);
      vbuf[i] = buffer_load16(rv, row * RB + col);
    }
  };
  auto store_tile = [&](int stage) __attribute__((always_inline)) {
    char FA_LDS* kt = ring + stage * 2 * TILE;
    char FA_LDS* vt = kt + TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int cidx = ptid + 128 * i;
      const int off = tile_offset<D>(cidx / CPR, cidx % CPR);
      lds_write16(kt, off, kbuf[i]);
      lds_write16(vt, off, vbuf[i]);
    }
  };

  // transposing-read coordinates (see cdna4.h)
  const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
  const int tr_key = (tg >> 1) * 4 + tr;
  const int tr_byte = (tq & 1) * 8;

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_ref = NEG_INF, l_run = 0.f;

  // One key tile.  Tiles with hidden pairs (edges, tiles past this wave's keys) have them set
  // to -inf in a branch around the mask alone, so the accumulators see one code path (no
  // register copies where paths join); c > 0 and a finite reference turn -inf into P = 0.
  auto tile = [&](const char FA_LDS* kt, const char FA_LDS* vt, int j0, bool masked)
      __attribute__((always_inline)) {
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const i16x8 kop =
            __builtin_bit_cast(i16x8, lds_read16(kt, tile_offset<D>(32 * mb + l32, 2 * ks + hi)));
        s[mb] = mfma32x32x16<BF16>(kop, qreg[ks], s[mb]);
      }
    if (masked) {
      keep_branch();
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = j0 + 32 * mb + 8 * (i >> 2) + 4 * hi + (i & 3);
          s[mb][i] = mk.visible(qi, j) ? s[mb][i] : NEG_INF;
        }
    }
    float ext = s[0][0];
#pragma unroll
    for (int e = 1; e < 32; ++e) ext = fmaxf(ext, s[e / 16][e % 16]);
    ext = max_with_partner(ext);
    const float m_tile = __builtin_isinf(ext) ? NEG_INF : ext * c;
    const float g = m_tile - m_ref;
    const float l_row = sum_with_partner(l_run);
    const bool heavy = exp2_fast(g + 4.f) > l_row;
    const bool move = (g > 0.f) & ((g > kTauS) | heavy);
    if (__any(move)) {
      const float alpha = move ? exp2_fast(m_ref - m_tile) : 1.f;   // 0 on a first tile
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_ref = move ? m_tile : m_ref;
    }
    const float neg_m = m_ref == NEG_INF ? 0.f : -m_ref;
    unsigned pk[2][8];
    float part_sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = exp2_fast(__builtin_fmaf(s[mb][i], c, neg_m));
        const float p1 = exp2_fast(__builtin_fmaf(s[mb][i + 1], c, neg_m));
        part_sum[(i >> 1) & 3] += p0 + p1;
        pk[mb][i >> 1] = pack2<BF16>(p0, p1);
      }
    l_run += (part_sum[0] + part_sum[1]) + (part_sum[2] + part_sum[3]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int key_a = 16 * kk + tr_key;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int chunk = 4 * db + 2 * (tg & 1) + (tq >> 1);
        const i16x4 lo = lds_read_tr(vt, tile_offset<D>(key_a, chunk) + tr_byte);
        const i16x4 hi4 = lds_read_tr(vt, tile_offset<D>(key_a + 8, chunk) + tr_byte);
        const i16x8 vop = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        const u32x4 pb = {pk[kk >> 1][4 * (kk & 1) + 0], pk[kk >> 1][4 * (kk & 1) + 1],
                          pk[kk >> 1][4 * (kk & 1) + 2], pk[kk >> 1][4 * (kk & 1) + 3]};
        oacc[db] = mfma32x32x16<BF16>(vop, __builtin_bit_cast(i16x8, pb), oacc[db]);
      }
    }
  };

  if (p_tiles > 0) {
    load_tile(p_begin);
    store_tile(0);
  }
  __syncthreads();
  int stage = 0;
  for (int it = 0; it < max_tiles; ++it) {   // the same count in every wave: shared barriers
    const int t = p_begin + it;
    const bool have = it < p_tiles, have_next = it + 1 < p_tiles;
    const char FA_LDS* kt = ring + stage * 2 * TILE;
    const char FA_LDS* vt = kt + TILE;
    if (have_next) load_tile(t + 1);
    const int j0 = t * kBcS;
    if (have) {   // past the part's tiles the stage holds no tile of it
      const bool live = wave_has_rows && j0 < wkey_hi && j0 + kBcS > wkey_lo;
      tile(kt, vt, j0, !(live && mk.all_visible(wq0, wq1, j0, j0 + kBcS)));
    }
    if (have_next) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
  }

  // ---- merge of the parts: each wave leaves its normalised O^T and its LSE (base 2) in LDS
  // (over the rings, no longer read after the last barrier)
  float* mo = (float*)lds_raw;                       // [WAVES][DB][16][64]
  float* ml = mo + S::WAVES * DB * 16 * 64;          // [WAVES][64]
  {
    const float l_tot = sum_with_partner(l_run);
    const bool live = l_tot > 0.f;
    const float inv = live ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) mo[((wave * DB + db) * 16 + i) * 64 + lane] = oacc[db][i] * inv;
    ml[wave * 64 + lane] = live ? m_ref + __builtin_log2f(l_tot) : NEG_INF;
  }
  __syncthreads();
  if (part == 0 && qi < n) {
    float lp[KSPLIT], lmax = NEG_INF;
#pragma unroll
    for (int p = 0; p < KSPLIT; ++p) {
      lp[p] = ml[(2 * p + stripe) * 64 + lane];
      lmax = fmaxf(lmax, lp[p]);
    }
    float wsum = 0.f, w[KSPLIT];
#pragma unroll
    for (int p = 0; p < KSPLIT; ++p) {
      w[p] = lmax == NEG_INF ? 0.f : exp2_fast(lp[p] - lmax);   // -inf parts weigh 0
      wsum += w[p];
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    char* orow = a.o + head + (long)qi * RB;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float r[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          float acc = 0.f;
#pragma unroll
          for (int p = 0; p < KSPLIT; ++p)
            acc += w[p] * mo[(((2 * p + stripe) * DB + db) * 16 + 4 * gq + x) * 64 + lane];
          r[x] = acc * inv;
        }
        const int dim = 32 * db + 8 * gq + 4 * hi;
        u32x2 v2 = {pack2<BF16>(r[0], r[1]), pack2<BF16>(r[2], r[3])};
        *reinterpret_cast<u32x2*>(orow + dim * 2) = v2;
      }
    if (a.lse != nullptr && hi == 0)
      a.lse[(long)bh * n + qi] = wsum > 0.f ? (lmax + __builtin_log2f(wsum)) * kLn2 : NEG_INF;
  }
}

template <int D, bool BF16>
hipError_t launch_s(const FwdParams& p, hipStream_t stream) {
  SplitArgs a;
  a.q = static_cast<const char*>(p.q);
  a.k = static_cast<const char*>(p.k);
  a.v = static_cast<const char*>(p.v);
  a.o = static_cast<char*>(p.o);
  a.lse = p.lse;
  a.n = p.N;
  a.n_bh = p.B * p.H;
  a.n_qt = (p.N + kBqS - 1) / kBqS;
  a.c = (float)(std::fmax(std::fabs((double)p.scale), 1e-30) * 1.4426950408889634);
  a.q_sign = p.scale < 0.f ? 0x80008000u : 0u;
  a.causal = p.causal;
  a.wl = p.window_left;
  a.wr = p.causal ? 0 : p.window_right;
  const long blocks = (long)a.n_bh * a.n_qt;
  hipLaunchKernelGGL((fwd_split_kernel<D, BF16>), dim3((unsigned)blocks),
                     dim3(SplitShape<D>::THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_split(const FwdParams& p, hipStream_t stream) {
  if (p.D == 64) return p.bf16 ? launch_s<64, true>(p, stream) : launch_s<64, false>(p, stream);
  return p.bf16 ? launch_s<128, true>(p, stream) : launch_s<128, false>(p, stream);
}

}  // namespace fa
