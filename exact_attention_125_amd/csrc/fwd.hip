// Fused attention forward for gfx950.
//
// One workgroup owns one tile of Br = 128 query rows of one (batch, head); each of its four
// waves owns 32 of those rows.  The key/value sequence streams through LDS in tiles of
// Bc = 64 keys, double-buffered: while the waves work on tile t, the loads of tile t+1 are
// already in flight into registers, and land in the other LDS buffer afterwards.  Per tile:
//
//   S^T = K Q^T        32x32x16 MFMAs, K from LDS (A operand), Q^T kept in registers
//   mask               only on tiles that straddle a causal/window/sequence edge; tiles
//                      that are hidden entirely are never visited
//   online softmax     running max m and running sum l per query, in base 2 with the
//                      scale folded into one FMA (x*scale*log2e - m)
//   O^T += V^T P^T     32x32x16 MFMAs, V^T read from LDS with transposing reads, P^T taken
//                      straight from the S^T accumulators (no LDS round trip)
//
// Computing the transposed score block puts one query in each lane (keys spread over the
// lane's registers and its partner lane l^32), so row max and row sum are in-lane
// reductions plus one permlane32 swap, and the rescale of O^T by exp(m_old - m_new) is a
// per-lane scalar.  The method follows the tiling of "告别OOM和训练慢：用Flash Attention加速
// 你的PyTorch大模型（含A100环境配置）" §2.1 and its running-max / running-sum update of §2.2
// (read as l_new = exp(m_old - m_new) l_old + sum exp(s - m_new), with O rescaled by the
// same factor and divided by l once at the end), and the per-query-block loop of
// "Flash Attention 3.7 核心原理与实战：加速Transformer模型训练与推理" §3.1.
#include <type_traits>

#include "cdna4.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kBr = 32 * kWaves;   // query rows per workgroup
constexpr int kBc = 64;            // keys per K/V tile

struct FwdArgs {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int n;          // sequence length
  int n_bh;       // batch * heads
  int n_qt;       // query tiles per head
  float c;        // softmax_scale * log2(e)
  int causal, wl, wr;
};

template <int D, bool BF16>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs a) {
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kBc * kRowBytes;
  constexpr int kChunks = D / 8;                    // 16-byte chunks per row
  constexpr int kLoads = kBc * kChunks / 256;       // chunks per thread per tile
  constexpr int kKs = D / 16;                       // MFMA k-steps over the head dim
  constexpr int kDb = D / 32;                       // 32-wide blocks of the head dim

  __shared__ __attribute__((aligned(16))) char lds_raw[2 * 2 * kTileBytes];
  char FA_LDS* lds = (char FA_LDS*)(lds_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, qt;
  xcd_tile_order(blockIdx.x, a.n_bh, a.n_qt, bh, qt);
  if (a.causal) qt = a.n_qt - 1 - qt;               // longest rows first
  const int n = a.n;
  const int q0 = qt * kBr;
  const long head = (long)bh * n * kRowBytes;
  const int head_bytes = n * kRowBytes;
  const auto rq = make_rsrc(a.q + head, head_bytes);
  const auto rk = make_rsrc(a.k + head, head_bytes);
  const auto rv = make_rsrc(a.v + head, head_bytes);

  // Q^T as the B operand: lane holds query (q0 + 32 wave + l32), head-dim chunk 2 ks + hi.
  const int qi = q0 + 32 * wave + l32;
  i16x8 qreg[kKs];
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks)
    qreg[ks] = __builtin_bit_cast(i16x8, buffer_load16(rq, qi * kRowBytes + (2 * ks + hi) * 16));

  const Mask mk{n, a.causal, a.wl, a.wr};
  const int q_last = q0 + kBr - 1;
  int key_lo, key_hi;
  mk.key_range(q0, min(q_last, n - 1), key_lo, key_hi);
  const int t_begin = key_lo / kBc;
  const int t_end = (key_hi + kBc - 1) / kBc;

  u32x4 kbuf[kLoads], vbuf[kLoads];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + 256 * i;
      const int off = (t * kBc + c / kChunks) * kRowBytes + (c % kChunks) * 16;
      kbuf[i] = buffer_load16(rk, off);
      vbuf[i] = buffer_load16(rv, off);
    }
  };
  auto store_tile = [&](int stage) {
    char FA_LDS* kt = lds + stage * 2 * kTileBytes;
    char FA_LDS* vt = kt + kTileBytes;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + 256 * i;
      const int off = tile_offset<D>(c / kChunks, c % kChunks);
      lds_write16(kt, off, kbuf[i]);
      lds_write16(vt, off, vbuf[i]);
    }
  };

  const float c = a.c;
  const float NEG_INF = -__builtin_inff();
  float m_run = NEG_INF;   // running max of the scaled scores, base-2 units
  float l_run = 0.f;       // running sum of 2^(s*c - m_run) over this lane's keys
  f32x16 oacc[kDb];
#pragma unroll
  for (int db = 0; db < kDb; ++db) oacc[db] = f32x16{};

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
  }
  __syncthreads();

  // Transposing-read coordinates of this lane (see cdna4.h): 16-lane group G, row r, quad t.
  const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
  const int tr_key = (tg >> 1) * 4 + tr;
  const int tr_byte = (tq & 1) * 8;

  // One key tile.  MASKED selects the variant for tiles that straddle an edge; the common
  // variant has no per-element work beyond the softmax itself.
  auto tile = [&](auto masked_tag, const char FA_LDS* kt, const char FA_LDS* vt, int j0) {
    constexpr bool MASKED = decltype(masked_tag)::value;

    // ---- S^T = K Q^T: two 32-key blocks x 32 queries
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        const i16x8 kop = __builtin_bit_cast(i16x8, lds_read16(kt, tile_offset<D>(32 * mb + l32, 2 * ks + hi)));
        s[mb] = mfma32x32x16<BF16>(kop, qreg[ks], s[mb]);
      }
    }

    unsigned vis_bits = 0xffffffffu;
    if constexpr (MASKED) {
      const float sentinel = c >= 0.f ? NEG_INF : __builtin_inff();
      vis_bits = 0;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = j0 + 32 * mb + 8 * (i >> 2) + 4 * hi + (i & 3);
          const bool ok = mk.visible(qi, j);
          vis_bits |= (ok ? 1u : 0u) << (16 * mb + i);
          s[mb][i] = ok ? s[mb][i] : sentinel;
        }
    }

    // ---- row extreme of the raw scores (max, or min for a negative scale)
    float ext;
    if (c >= 0.f) {
      ext = NEG_INF;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) ext = fmaxf(ext, s[mb][i]);
      ext = max_with_partner(ext);
    } else {
      ext = __builtin_inff();
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) ext = fminf(ext, s[mb][i]);
      ext = min_with_partner(ext);
    }
    const float m_tile = __builtin_isinf(ext) ? NEG_INF : ext * c;

    // ---- running max: the reference moves to the exact row max whenever it grows, so the
    // largest probability of a row is exactly 1 (representable in every input type).  O
    // and l are rescaled only when some row of the wave actually grew.
    const float m_new = fmaxf(m_run, m_tile);
    if (__any(m_new > m_run)) {
      // alpha = 1 for rows that did not grow (also rows with no visible key yet, where
      // m_run - m_new would be -inf - -inf); 0 for a row's first visible key
      const float alpha = m_new > m_run ? exp2_fast(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < kDb; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float neg_m = m_run == NEG_INF ? 0.f : -m_run;

    // P = 2^(s*c - m); l accumulates the unrounded values in fp32 (the logsumexp keeps full
    // precision), P itself is rounded once to the input type for the P.V product.
    unsigned pk[2][8];
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float p0 = exp2_fast(__builtin_fmaf(s[mb][i], c, neg_m));
        float p1 = exp2_fast(__builtin_fmaf(s[mb][i + 1], c, neg_m));
        if constexpr (MASKED) {
          p0 = (vis_bits >> (16 * mb + i)) & 1u ? p0 : 0.f;
          p1 = (vis_bits >> (16 * mb + i + 1)) & 1u ? p1 : 0.f;
        }
        part[(i >> 1) & 3] += p0 + p1;
        pk[mb][i >> 1] = pack2<BF16>(p0, p1);
      }
    l_run += (part[0] + part[1]) + (part[2] + part[3]);

    // ---- O^T += V^T P^T
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 pb = {pk[kk >> 1][4 * (kk & 1) + 0], pk[kk >> 1][4 * (kk & 1) + 1],
                        pk[kk >> 1][4 * (kk & 1) + 2], pk[kk >> 1][4 * (kk & 1) + 3]};
      const int key_a = 16 * kk + tr_key;
#pragma unroll
      for (int db = 0; db < kDb; ++db) {
        const int chunk = 4 * db + 2 * (tg & 1) + (tq >> 1);
        const i16x4 lo = lds_read_tr(vt, tile_offset<D>(key_a, chunk) + tr_byte);
        const i16x4 hi4 = lds_read_tr(vt, tile_offset<D>(key_a + 8, chunk) + tr_byte);
        const i16x8 vop = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = mfma32x32x16<BF16>(vop, __builtin_bit_cast(i16x8, pb), oacc[db]);
      }
    }
  };

  for (int t = t_begin; t < t_end; ++t) {
    const int stage = (t - t_begin) & 1;
    const char FA_LDS* kt = lds + stage * 2 * kTileBytes;
    const char FA_LDS* vt = kt + kTileBytes;
    if (t + 1 < t_end) load_tile(t + 1);
    const int j0 = t * kBc;
    if (mk.all_visible(q0, q_last, j0, j0 + kBc))
      tile(std::false_type{}, kt, vt, j0);
    else
      tile(std::true_type{}, kt, vt, j0);
    if (t + 1 < t_end) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l)
  const float l_tot = sum_with_partner(l_run);
  if (qi < n) {
    const float inv = 1.f / l_tot;
    char* orow = a.o + head + (long)qi * kRowBytes;
#pragma unroll
    for (int db = 0; db < kDb; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = 32 * db + 8 * g + 4 * hi;
        u32x2 w = {pack2<BF16>(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                   pack2<BF16>(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + dim * 2) = w;
      }
    if (a.lse != nullptr && hi == 0)
      a.lse[(long)bh * n + qi] = (m_run + __builtin_log2f(l_tot)) * kLn2;
  }
}

template <int D, bool BF16>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  FwdArgs a;
  a.q = static_cast<const char*>(p.q);
  a.k = static_cast<const char*>(p.k);
  a.v = static_cast<const char*>(p.v);
  a.o = static_cast<char*>(p.o);
  a.lse = p.lse;
  a.n = p.N;
  a.n_bh = p.B * p.H;
  a.n_qt = (p.N + kBr - 1) / kBr;
  a.c = (float)((double)p.scale * 1.4426950408889634);
  a.causal = p.causal;
  a.wl = p.window_left;
  a.wr = p.causal ? 0 : p.window_right;   // causal is a right bound of 0
  const long blocks = (long)a.n_bh * a.n_qt;
  hipLaunchKernelGGL((fwd_kernel<D, BF16>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  if (p.D == 64) return p.bf16 ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return p.bf16 ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace fa
