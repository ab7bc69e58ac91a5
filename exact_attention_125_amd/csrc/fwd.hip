// Fused attention forward for gfx950.
//
// One workgroup owns Br = 32 * QB * WAVES query rows of one (batch, head); each wave owns
// 32 * QB of them (QB query blocks of 32).  The key/value sequence streams through LDS in
// tiles of Bc = 64 keys, double-buffered: while the waves work on tile t, the loads of tile
// t+1 are in flight into registers and land in the other LDS buffer afterwards.  Per tile
// and wave:
//
//   S^T = K Q^T        32x32x16 MFMAs; each K operand read from LDS feeds QB MFMAs (one
//                      per query block), Q^T stays in registers for the whole loop
//   mask               only on tiles that straddle a causal/window/sequence edge for this
//                      wave; tiles hidden from all of the wave's queries are skipped
//   online softmax     a per-query reference m (base 2, scale folded into one FMA
//                      x*c - m); P = 2^(x*c - m), l += P in fp32, P rounded once to the
//                      input type
//   O^T += V^T P^T     32x32x16 MFMAs, V^T read from LDS with transposing reads (each
//                      feeds QB MFMAs), P^T taken straight from the S^T accumulators
//
// Computing the transposed score block puts one query in each lane (keys spread over the
// lane's registers and its partner lane l^32), so row max and row sum are in-lane
// reductions plus one permlane32 swap, and rescaling O^T is a per-lane scalar multiply.
//
// The method is the tiling of "告别OOM和训练慢：用Flash Attention加速你的PyTorch大模型（含A100环境
// 配置）" §2.1 with the running-max / running-sum update of its §2.2 (read as
// l_new = exp(m_old - m_new) l_old + sum exp(s - m_new), O rescaled by the same factor and
// divided by l once at the end), looping over key blocks per query block as "Flash
// Attention 3.7 核心原理与实战：加速Transformer模型训练与推理" §3.1 describes.
//
// The reference m of a query is the exact maximum of its first visible tile.  A later tile
// whose maximum exceeds m by g > 0 moves m to that exact maximum (rescaling O and l) unless
// the new largest probability 2^g is small against the mass already summed (2^g * 16 <= l)
// and g <= kTau.  The softmax does not depend on the shift (the safe-softmax argument of the
// same §2.2), so the result is the same up to rounding; probabilities stay at most 2^kTau,
// which every input type represents.  Rows dominated by a few keys still get their exact
// maximum (a probability of exactly 1, exact in every input type), while on long rows the
// O/l rescale, a multiply per accumulator, disappears from almost every tile.  The
// logsumexp is m + log2(l) whatever m is.
//
// A negative softmax scale is handled exactly by flipping the sign bits of Q in registers
// (s * scale = (-q).k * |scale|), so the kernel only ever needs row maxima.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "cdna4.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kBc = 64;           // keys per K/V tile
constexpr float kTau = 8.0f;      // largest lag (base 2) of the reference behind a row max

struct FwdArgs {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  long long q_bs, q_hs, k_bs, k_hs, v_bs, v_hs, o_bs, o_hs;   // batch / head strides, bytes
  int q_rs, k_rs, v_rs, o_rs;                                 // row strides, bytes
  int nq, nk;     // query rows, key rows
  int off;        // key position of query 0 (nk - nq)
  int n_h;        // heads
  int n_bh;       // batch * heads
  int n_qt;       // query tiles per head
  int n_split;    // key splits: each workgroup sees only its split's key tiles
  int split_tiles;  // key tiles per split
  float* po;      // n_split > 1: normalised partial O, fp32 [n_split, B*H, nq, D]
  float* plse;    //              and its natural-log LSE [n_split, B*H, nq]
  const float* slopes;   // ALiBi slopes [heads] (device), read by the ALIBI instances only
  Dropout drop;          // used by the DROPOUT instances only
  const unsigned char* blocks;   // block-sparse mask [heads][n_qb][n_kb] of 64 x 64 blocks, or null
  const unsigned char* kpm;      // key padding mask [batch][nk] (nonzero = padding key), or null
  int n_qb, n_kb;
  float c;        // |softmax_scale| * log2(e)
  unsigned q_sign;  // 0x80008000 to negate Q (negative scale), else 0
  int causal, wl, wr;
};

// Buffer resource over the rows [0, rows) of one operand with a row stride of rs bytes: the
// last row ends after its D elements, so every row at or past `rows` reads as zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const char* base, int rows, int rs,
                                                            int row_bytes) {
  return make_rsrc(base, rows > 0 ? (rows - 1) * rs + row_bytes : 0);
}

// ALIBI: every score gets the ALiBi penalty -slope_h |p - j| (p the query's key position), in
// the exponent domain: s <- s c - slope log2(e) |p - j| right after the product, after which
// the tile works with a unit factor in place of c.
// DROPOUT: the weights that multiply V are P * keep * drop.scale, drop.scale the inverse of the
// keep probability (the row sums stay those of P),
// with keep drawn by a.drop.
template <int D, bool BF16, int WAVES, int QB, bool ALIBI, bool DROPOUT>
__global__ __launch_bounds__(64 * WAVES, (D == 64 ? 2 : 1)) void fwd_kernel(FwdArgs a) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kBr = 32 * QB * WAVES;
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kBc * kRowBytes;
  constexpr int kChunks = D / 8;                      // 16-byte chunks per row
  constexpr int kLoads = kBc * kChunks / kThreads;    // chunks per thread per tile (K or V)
  constexpr int kKs = D / 16;                         // MFMA k-steps over the head dim
  constexpr int kDb = D / 32;                         // 32-wide blocks of the head dim
  static_assert(kBc * kChunks % kThreads == 0, "tile must split evenly over the threads");

  __shared__ __attribute__((aligned(16))) char lds_raw[2 * 2 * kTileBytes];
  char FA_LDS* lds = (char FA_LDS*)(lds_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, slot;
  xcd_tile_order(blockIdx.x, a.n_bh, a.n_qt * a.n_split, bh, slot);
  int qt = slot / a.n_split;
  const int split = slot - qt * a.n_split;
  if (a.causal) qt = a.n_qt - 1 - qt;               // longest rows first
  const int nq = a.nq, nk = a.nk, off = a.off;
  const int q0 = qt * kBr;
  const int b = bh / a.n_h, h = bh - b * a.n_h;
  const auto rq = rows_rsrc(a.q + b * a.q_bs + h * a.q_hs, nq, a.q_rs, kRowBytes);
  const auto rk = rows_rsrc(a.k + b * a.k_bs + h * a.k_hs, nk, a.k_rs, kRowBytes);
  const auto rv = rows_rsrc(a.v + b * a.v_bs + h * a.v_hs, nk, a.v_rs, kRowBytes);

  // This wave's queries: block qb holds query wq0 + 32 qb + l32 in lane l.  Query i sits at
  // key position i + off; the mask works on positions.
  const int wq0 = q0 + 32 * QB * wave;
  const int wq1 = wq0 + 32 * QB - 1;
  // block-sparse: this wave's row of the block mask (its queries lie in one 64-query block;
  // a key tile is one 64-key block)
  static_assert(32 * QB <= 64 && kBc == 64, "a wave's tile lies in one 64 x 64 block");
  const unsigned char* brow =
      a.blocks ? a.blocks + ((long)h * a.n_qb + wq0 / 64) * a.n_kb : nullptr;
  // key padding: this batch entry's row of the mask
  const unsigned char* kpm = a.kpm ? a.kpm + (long)b * nk : nullptr;

  // Q^T as the B operand: lane holds query (wq0 + 32 qb + l32), head-dim chunk 2 ks + hi.
  i16x8 qreg[QB][kKs];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      u32x4 x = buffer_load16(rq, (wq0 + 32 * qb + l32) * a.q_rs + (2 * ks + hi) * 16);
      x ^= a.q_sign;
      qreg[qb][ks] = __builtin_bit_cast(i16x8, x);
    }

  const Mask mk{nk, a.causal, a.wl, a.wr};
  int key_lo, key_hi;
  mk.key_range(q0 + off, min(q0 + kBr - 1, nq - 1) + off, key_lo, key_hi);
  // this split's share of the key tiles
  const int t_begin = max(max(key_lo, 0) / kBc, split * a.split_tiles);
  const int t_end = min((max(key_hi, 0) + kBc - 1) / kBc, (split + 1) * a.split_tiles);
  // The keys this wave's own queries can see (tiles outside are skipped by this wave).
  int wkey_lo, wkey_hi;
  mk.key_range(wq0 + off, min(wq1, nq - 1) + off, wkey_lo, wkey_hi);
  const bool wave_has_rows = wq0 < nq;

  u32x4 kbuf[kLoads], vbuf[kLoads];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + kThreads * i;
      const int row = t * kBc + c / kChunks, col = (c % kChunks) * 16;
      kbuf[i] = buffer_load16(rk, row * a.k_rs + col);
      vbuf[i] = buffer_load16(rv, row * a.v_rs + col);
    }
  };
  auto store_tile = [&](int stage) {
    char FA_LDS* kt = lds + stage * 2 * kTileBytes;
    char FA_LDS* vt = kt + kTileBytes;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + kThreads * i;
      const int off = tile_offset<D>(c / kChunks, c % kChunks);
      lds_write16(kt, off, kbuf[i]);
      lds_write16(vt, off, vbuf[i]);
    }
  };

  const float c = ALIBI ? 1.f : a.c;   // the ALIBI instances scale the scores in place
  const float b2 = ALIBI ? a.slopes[h] * kLog2e : 0.f;
  const float NEG_INF = -__builtin_inff();
  float m_ref[QB];      // reference of the exponent per query, base-2 units
  float l_run[QB];      // sum of 2^(s*c - m_ref) over this lane's keys
  f32x16 oacc[kDb][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = NEG_INF;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < kDb; ++db) oacc[db][qb] = f32x16{};
  }

  // Block-sparse: the workgroup visits only the key tiles that one of its two 64-query
  // block rows selects (the others are neither loaded nor waited for).
  const unsigned char* wg_row0 =
      a.blocks ? a.blocks + ((long)h * a.n_qb + q0 / 64) * a.n_kb : nullptr;
  const unsigned char* wg_row1 =
      (a.blocks && q0 / 64 + 1 < a.n_qb) ? wg_row0 + a.n_kb : wg_row0;
  auto next_tile = [&](int t) {   // first visited tile at or after t
    if (wg_row0 != nullptr)
      while (t < t_end && !(wg_row0[t] | wg_row1[t])) ++t;
    return t;
  };
  const int t_first = next_tile(t_begin);
  if (t_first < t_end) {
    load_tile(t_first);
    store_tile(0);
  }
  __syncthreads();

  // Transposing-read coordinates of this lane (see cdna4.h): 16-lane group G, row r, quad t.
  const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
  const int tr_key = (tg >> 1) * 4 + tr;
  const int tr_byte = (tq & 1) * 8;

  // One key tile for this wave.  MASKED selects the variant for tiles that straddle an
  // edge or hold padding keys (bit j - j0 of pad set); the common variant has no per-element
  // work beyond the softmax itself.
  // (Tiles with hidden pairs have them set to -inf in a branch around the mask alone, so the
  // accumulators see one code path, with no register copies where paths join.)
  auto tile = [&](const char FA_LDS* kt, const char FA_LDS* vt, int j0, unsigned long long pad,
                  bool masked) {

    // ---- S^T = K Q^T: two 32-key blocks x QB query blocks
    f32x16 s[2][QB];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[mb][qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const i16x8 kop =
            __builtin_bit_cast(i16x8, lds_read16(kt, tile_offset<D>(32 * mb + l32, 2 * ks + hi)));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[mb][qb] = mfma32x32x16<BF16>(kop, qreg[qb][ks], s[mb][qb]);
      }

    if constexpr (ALIBI) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qpos = wq0 + 32 * qb + l32 + off;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = j0 + 32 * mb + 8 * (i >> 2) + 4 * hi + (i & 3);
            s[mb][qb][i] = __builtin_fmaf(s[mb][qb][i], a.c, -b2 * __builtin_fabsf((float)(qpos - j)));
          }
      }
    }

    if (masked) {
      keep_branch();
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qpos = wq0 + 32 * qb + l32 + off;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int t = 32 * mb + 8 * (i >> 2) + 4 * hi + (i & 3);
            const bool vis = mk.visible(qpos, j0 + t) && ((pad >> t) & 1ull) == 0;
            s[mb][qb][i] = vis ? s[mb][qb][i] : NEG_INF;
          }
      }
    }

    // ---- tile maximum per query; move the reference where the new maximum matters.
    // Both lanes of a query (l and l^32) see the same m_tile and the same full-row sum, so
    // they always take the same decision.
    float m_tile[QB];
    bool move[QB];
    bool move_any = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float ext = s[0][qb][0];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = (mb == 0 ? 1 : 0); i < 16; ++i) ext = fmaxf(ext, s[mb][qb][i]);
      ext = max_with_partner(ext);
      m_tile[qb] = __builtin_isinf(ext) ? NEG_INF : ext * c;
      // g = +inf on a row's first visible tile (m_ref = -inf); NaN or -inf (no visible key
      // in this tile) compares false
      const float g = m_tile[qb] - m_ref[qb];
      const float l_row = sum_with_partner(l_run[qb]);   // all lanes take part
      const bool heavy = exp2_fast(g + 4.f) > l_row;
      move[qb] = (g > 0.f) & ((g > kTau) | heavy);   // no short-circuit branches
      move_any |= move[qb];
    }
    if (__any(move_any)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const bool grow = move[qb];
        // the first visible tile of a row has m_ref = -inf: alpha = 0 (nothing to keep)
        const float alpha = grow ? exp2_fast(m_ref[qb] - m_tile[qb]) : 1.f;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < kDb; ++db) oacc[db][qb] *= alpha;
        m_ref[qb] = grow ? m_tile[qb] : m_ref[qb];
      }
    }

    // ---- P = 2^(s*c - m); l accumulates the unrounded values in fp32 (the logsumexp keeps
    // full precision), P itself is rounded once to the input type for the P.V product.
    unsigned pk[QB][2][8];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float neg_m = m_ref[qb] == NEG_INF ? 0.f : -m_ref[qb];
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        unsigned rw[4][2];   // DROPOUT: this query's draws for the block's four runs of keys
        if constexpr (DROPOUT) a.drop.runs4(bh, wq0 + 32 * qb + l32, j0 + 32 * mb + 4 * hi, rw);
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          // hidden scores are -inf: with c > 0 (a zero scale is kept tiny) and a finite
          // reference shift they give 2^-inf = 0
          float p0 = exp2_fast(__builtin_fmaf(s[mb][qb][i], c, neg_m));
          float p1 = exp2_fast(__builtin_fmaf(s[mb][qb][i + 1], c, neg_m));
          part[(i >> 1) & 3] += p0 + p1;
          if constexpr (DROPOUT) {   // keys j, j + 1: the low and high half of one word
            const unsigned w = rw[i >> 2][(i & 3) >> 1];
            p0 = a.drop.keep_half(w, 0) ? p0 * a.drop.scale : 0.f;
            p1 = a.drop.keep_half(w, 1) ? p1 * a.drop.scale : 0.f;
          }
          pk[qb][mb][i >> 1] = pack2<BF16>(p0, p1);
        }
      }
      l_run[qb] += (part[0] + part[1]) + (part[2] + part[3]);
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int key_a = 16 * kk + tr_key;
#pragma unroll
      for (int db = 0; db < kDb; ++db) {
        const int chunk = 4 * db + 2 * (tg & 1) + (tq >> 1);
        const i16x4 lo = lds_read_tr(vt, tile_offset<D>(key_a, chunk) + tr_byte);
        const i16x4 hi4 = lds_read_tr(vt, tile_offset<D>(key_a + 8, chunk) + tr_byte);
        const i16x8 vop = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const u32x4 pb = {pk[qb][kk >> 1][4 * (kk & 1) + 0], pk[qb][kk >> 1][4 * (kk & 1) + 1],
                            pk[qb][kk >> 1][4 * (kk & 1) + 2], pk[qb][kk >> 1][4 * (kk & 1) + 3]};
          oacc[db][qb] = mfma32x32x16<BF16>(vop, __builtin_bit_cast(i16x8, pb), oacc[db][qb]);
        }
      }
    }
  };

  int stage = 0;
  for (int t = t_first; t < t_end;) {
    const char FA_LDS* kt = lds + stage * 2 * kTileBytes;
    const char FA_LDS* vt = kt + kTileBytes;
    const int t_next = next_tile(t + 1);
    if (t_next < t_end) load_tile(t_next);
    const int j0 = t * kBc;
    // key padding: bit i of pad marks key j0 + i as padding (keys past nk count as padding
    // here; the sequence mask hides them anyway)
    unsigned long long pad = 0;
    if (kpm != nullptr) pad = __ballot(j0 + lane >= nk || kpm[j0 + lane] != 0);
    if (wave_has_rows && j0 < wkey_hi && j0 + kBc > wkey_lo && (brow == nullptr || brow[t]) &&
        pad != ~0ull)
      tile(kt, vt, j0, pad, !(pad == 0 && mk.all_visible(wq0 + off, wq1 + off, j0, j0 + kBc)));
    if (t_next < t_end) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    t = t_next;
  }

  // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l); a row that saw no key (possible
  // only with nq != nk or a key split) gets O = 0 and LSE = -inf
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = wq0 + 32 * qb + l32;
    const float l_tot = sum_with_partner(l_run[qb]);
    if (qi < nq) {
      const bool live = l_tot > 0.f;
      const float inv = live ? 1.f / l_tot : 0.f;
      const float lse = live ? (m_ref[qb] + __builtin_log2f(l_tot)) * kLn2 : NEG_INF;
      if (a.n_split == 1) {
        char* orow = a.o + b * a.o_bs + h * a.o_hs + (long)qi * a.o_rs;
#pragma unroll
        for (int db = 0; db < kDb; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int dim = 32 * db + 8 * g + 4 * hi;
            u32x2 w = {pack2<BF16>(oacc[db][qb][4 * g + 0] * inv, oacc[db][qb][4 * g + 1] * inv),
                       pack2<BF16>(oacc[db][qb][4 * g + 2] * inv, oacc[db][qb][4 * g + 3] * inv)};
            *reinterpret_cast<u32x2*>(orow + dim * 2) = w;
          }
        if (a.lse != nullptr && hi == 0) a.lse[(long)bh * nq + qi] = lse;
      } else {
        const long prow = ((long)split * a.n_bh + bh) * nq + qi;
        float* po = a.po + prow * D;
#pragma unroll
        for (int db = 0; db < kDb; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int dim = 32 * db + 8 * g + 4 * hi;
            const f32x4 w = {oacc[db][qb][4 * g + 0] * inv, oacc[db][qb][4 * g + 1] * inv,
                             oacc[db][qb][4 * g + 2] * inv, oacc[db][qb][4 * g + 3] * inv};
            *reinterpret_cast<f32x4*>(po + dim) = w;
          }
        if (hi == 0) a.plse[prow] = lse;
      }
    }
  }
}

template <int D, bool BF16, int WAVES, int QB>
hipError_t launch_args(FwdArgs& a, hipStream_t stream) {
  constexpr int kBr = 32 * QB * WAVES;
  a.n_qt = (a.nq + kBr - 1) / kBr;
  const long blocks = (long)a.n_bh * a.n_qt * a.n_split;
  const dim3 grid((unsigned)blocks), block(64 * WAVES);
  const bool alibi = a.slopes != nullptr, drop = a.drop.scale != 1.f;
  if (alibi && drop)
    hipLaunchKernelGGL((fwd_kernel<D, BF16, WAVES, QB, true, true>), grid, block, 0, stream, a);
  else if (alibi)
    hipLaunchKernelGGL((fwd_kernel<D, BF16, WAVES, QB, true, false>), grid, block, 0, stream, a);
  else if (drop)
    hipLaunchKernelGGL((fwd_kernel<D, BF16, WAVES, QB, false, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_kernel<D, BF16, WAVES, QB, false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

void set_mask_and_scale(FwdArgs& a, float scale, int causal, int wl, int wr) {
  // a zero scale becomes a tiny one: every visible probability is then exactly 1 (as for 0)
  // while hidden scores (-inf) still give 0 instead of -inf * 0 = NaN
  a.c = (float)(std::fmax(std::fabs((double)scale), 1e-30) * 1.4426950408889634);
  a.q_sign = scale < 0.f ? 0x80008000u : 0u;
  a.causal = causal;
  a.wl = wl;
  a.wr = causal ? 0 : wr;   // causal is a right bound of 0
}

template <int D, bool BF16, int WAVES, int QB>
hipError_t launch_cfg(const FwdParams& p, hipStream_t stream) {
  constexpr long kRow = (long)D * 2;
  FwdArgs a;
  a.q = static_cast<const char*>(p.q);
  a.k = static_cast<const char*>(p.k);
  a.v = static_cast<const char*>(p.v);
  a.o = static_cast<char*>(p.o);
  a.lse = p.lse;
  a.q_hs = a.k_hs = a.v_hs = a.o_hs = (long long)p.N * kRow;
  a.q_bs = a.k_bs = a.v_bs = a.o_bs = (long long)p.H * p.N * kRow;
  a.q_rs = a.k_rs = a.v_rs = a.o_rs = (int)kRow;
  a.nq = a.nk = p.N;
  a.off = 0;
  a.n_h = p.H;
  a.n_bh = p.B * p.H;
  a.n_split = 1;
  a.split_tiles = (p.N + kBc - 1) / kBc;
  a.po = a.plse = nullptr;
  a.slopes = nullptr;
  a.drop = Dropout{0u, 0u, 0u, 0u, 1.f};
  a.blocks = nullptr;
  a.kpm = nullptr;
  a.n_qb = a.n_kb = 0;
  set_mask_and_scale(a, p.scale, p.causal, p.window_left, p.window_right);
  return launch_args<D, BF16, WAVES, QB>(a, stream);
}

// Four waves of 32 query rows per workgroup: 128-row workgroups, twice as many as the
// 8-wave kernel's, for grids too small to fill the chip with those.
template <int D, bool BF16>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  return launch_cfg<D, BF16, 4, 1>(p, stream);
}

static_assert(kBc == kKvMfmaKeyStep, "key splits of the MFMA kernel are whole key tiles");

// Kernel requested through the environment (FA_FWD_KERNEL = "main" or "basic"), 0 if unset.
// A tuning and testing knob, read at every call and ignored unless set.
int env_kernel_choice() {
  const char* e = std::getenv("FA_FWD_KERNEL");
  if (e == nullptr) return 0;
  if (std::strcmp(e, "main") == 0) return 1;
  if (std::strcmp(e, "basic") == 0) return 2;
  if (std::strcmp(e, "split") == 0) return 3;
  return 0;
}

}  // namespace

// The main kernel (128 query rows per workgroup, two workgroups per CU) fills the chip when
// there are at least two 128-row query tiles per CU, i.e. B H ceil(N / 256) >= 256.  Smaller
// grids split the key loop over the waves of a workgroup (fwd_split.hip: 64 query rows, 2 to 4
// key parts), as long as there are keys enough to split (N >= 256); the shortest sequences
// run the four-wave kernel.  FA_FWD_KERNEL=main|basic|split forces one of them.
hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  const long pp_blocks = (long)p.B * p.H * ((p.N + 255) / 256);
  int choice = env_kernel_choice();
  if (choice == 0) choice = pp_blocks >= 256 ? 1 : (p.N >= 256 ? 3 : 2);
  if (p.seqlens != nullptr || p.cu != nullptr) choice = 1;   // padded / packed batches: main kernel
  if (choice == 1) return launch_fwd_main(p, stream);
  if (choice == 3) return launch_fwd_split(p, stream);
  if (p.D == 64) return p.bf16 ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return p.bf16 ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

// N_q queries over N_k keys on the four-wave kernel, with any strides and plan.n_split key
// splits (partial results into p.ws, merged afterwards by the caller's combine launch).
hipError_t launch_fwd_kv_mfma(const KvParams& p, const KvPlan& plan, hipStream_t stream) {
  const long long e = 2;   // bytes per element
  FwdArgs a;
  a.q = static_cast<const char*>(p.q);
  a.k = static_cast<const char*>(p.k);
  a.v = static_cast<const char*>(p.v);
  a.o = static_cast<char*>(p.o);
  a.lse = p.lse;
  a.q_bs = p.sq.b * e, a.q_hs = p.sq.h * e, a.q_rs = (int)(p.sq.r * e);
  a.k_bs = p.sk.b * e, a.k_hs = p.sk.h * e, a.k_rs = (int)(p.sk.r * e);
  a.v_bs = p.sv.b * e, a.v_hs = p.sv.h * e, a.v_rs = (int)(p.sv.r * e);
  a.o_bs = p.so.b * e, a.o_hs = p.so.h * e, a.o_rs = (int)(p.so.r * e);
  a.nq = p.Nq;
  a.nk = p.Nk;
  a.off = p.Nk - p.Nq;
  a.n_h = p.H;
  a.n_bh = p.B * p.H;
  a.n_split = plan.n_split;
  a.split_tiles = plan.split_keys / kBc;
  a.po = p.ws;
  a.plse = p.ws ? p.ws + (size_t)plan.n_split * a.n_bh * p.Nq * p.D : nullptr;
  a.slopes = p.slopes;
  a.drop = p.drop;
  a.blocks = p.blocks;
  a.kpm = p.kpm;
  a.n_qb = (p.Nq + 63) / 64;
  a.n_kb = (p.Nk + 63) / 64;
  set_mask_and_scale(a, p.scale, p.causal, p.window_left, p.window_right);
  if (p.D == 64)
    return p.bf16 ? launch_args<64, true, 4, 1>(a, stream) : launch_args<64, false, 4, 1>(a, stream);
  return p.bf16 ? launch_args<128, true, 4, 1>(a, stream) : launch_args<128, false, 4, 1>(a, stream);
}

}  // namespace fa
