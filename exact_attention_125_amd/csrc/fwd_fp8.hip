// Fused attention forward with FP8 E4M3 queries, keys and values for gfx950.
//
// Q, K and V arrive as E4M3 codes with one descale factor per tensor; both products run on
// the FP8 matrix instruction v_mfma_f32_32x32x64_f8f6f4 (fp32 accumulation), twice the rate
// of the 16-bit one.  A workgroup of 4 waves owns 128 query rows of one (batch, head), 32 per
// wave; key tiles of 64 keys stream through a double-buffered LDS stage (global loads into
// registers, written to the other buffer while the current tile is computed).  Per key tile
// and wave:
//
//   S^T = K Q^T           one FP8 product per 32 keys and 64 head dims; the K operand is one
//                         key row's 32 consecutive bytes (two 16-byte LDS reads), Q^T stays in
//                         registers
//   mask                  on tiles that straddle a causal / window / sequence edge
//   online softmax        reference m per query (base 2, the scale and both descales folded
//                         into one factor), P'' = 2^(s c - m + kPS), l += P'' in fp32
//   O^T += V^T P''^T      one FP8 product per 32 head dims: P'' is rounded once to E4M3 and
//                         taken straight from the S^T accumulators' registers; V^T comes from
//                         8-bit transposing LDS reads
//
// Lane layouts (checked on the device with one-hot operands): in the 32x32x64 FP8 product
// lane l supplies A[m = l % 32][k = 32 (l / 32) + e] and B[k = 32 (l / 32) + e][n = l % 32] as
// byte e = 0..31 of its eight registers, and C has the layout of the 16-bit products.  An
// S^T accumulator register i of 32-key block mb holds, in lane l, key 32 mb + 8 (i / 4) +
// 4 (l / 32) + i % 4 of query l % 32; the contraction index of the P V product is free, so
// byte e = 16 mb + i of a lane's B operand is that key, and the V^T operand supplies the
// same keys in the same byte order.  ds_read_b64_tr_b8: in each 16-lane group, lanes 2r and
// 2r + 1 address the two halves of a 16-byte row r (r = 0..7) and lane t receives byte t of
// rows 0..7; with the rows pointed at keys 16 rd + 8 (r / 4) + 4 (l / 32) + r % 4 (read rd =
// 0..3) and the 16 bytes at head dims 32 db + 16 (group % 2) .. + 15, lane l receives head
// dim 32 db + l % 32 of exactly the keys of its bytes 8 rd .. 8 rd + 7.
//
// Scaling of P: E4M3 is normal from 2^-6 to 448.  The reference lags the row maximum by at
// most kTau, so P = 2^(s c - m) <= 2^kTau; it enters the product as P'' = 2^kPS P <= 2^(kTau +
// kPS) = 256, normal down to P = 2^(-6 - kPS).  l sums the unrounded P'' and the factor
// cancels in O = acc / l; the logsumexp removes it.
//
// The arithmetic is the tiling of "告别OOM和训练慢：用Flash Attention加速你的PyTorch大模型
// （含A100环境配置）" §2.1 with the running max / running sum of its §2.2, as in the 16-bit
// kernels; FP8 is one of the next steps that page lists (§6).
#include <cmath>
#include <type_traits>

#include "cdna4.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kW8 = 4;              // waves per workgroup
constexpr int kT8 = 64 * kW8;       // threads per workgroup
constexpr int kBr8 = 32 * kW8;      // query rows per workgroup
constexpr int kBc8 = 64;            // keys per tile
constexpr float kTau8 = 4.0f;       // largest lag (base 2) of the reference behind a row max
constexpr float kPS = 4.0f;         // P enters the FP8 product as 2^kPS P

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

struct Fp8Args {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int n;          // rows per (batch, head)
  int n_bh;       // batch * heads
  int n_qt;       // query tiles per head
  int n_units;    // workgroups per head: n_qt, or ceil(n_qt / 2) query-tile pairs
  int paired;     // a workgroup takes query tiles u and n_qt - 1 - u
  float c;        // max(|softmax_scale|, tiny) * q_descale * k_descale * log2(e)
  float v_scale;  // v_descale
  unsigned q_sign;  // 0x80808080 negates Q (negative scale)
  int causal, wl, wr;
};

// The 16-byte chunk of a row that holds logical chunk `chunk`: an XOR with a function of the
// row, so that 16 consecutive rows at one chunk (K operand reads) and the 8 rows x 16 bytes of
// a transposing read fall into distinct banks.
template <int D>
__device__ __forceinline__ int swz8(int row) {
  if constexpr (D == 64)
    return (row >> 2) & 3;
  else
    return (row >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int tile_off8(int row, int chunk) {   // bytes
  return row * D + ((chunk ^ swz8<D>(row)) << 4);
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // E4M3 operands (format 0 for both), no block scaling
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// four fp32 values -> four E4M3 codes in one register (round to nearest even)
__device__ __forceinline__ int pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int D, bool BF16OUT>
__global__ __launch_bounds__(kT8, D == 64 ? 4 : 3) void fwd_fp8_kernel(Fp8Args a) {
  constexpr int RB = D;                         // bytes per row (one byte per element)
  constexpr int TILE = kBc8 * RB;               // bytes per K or V tile
  constexpr int CPR = D / 16;                   // 16-byte chunks per row
  constexpr int CPT = TILE / (16 * kT8);        // chunks per thread per tile (K or V)
  constexpr int KS = D / 64;                    // k-steps of the S product
  constexpr int DB = D / 32;                    // 32-dim blocks of O^T
  static_assert(CPT * 16 * kT8 == TILE, "whole chunks per thread");

  __shared__ __attribute__((aligned(16))) char lds_raw[2 * 2 * TILE];
  char FA_LDS* lds = (char FA_LDS*)lds_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, unit;
  xcd_tile_order(blockIdx.x, a.n_bh, a.n_units, bh, unit);
  const int n = a.n;
  const long head = (long)bh * n * RB;
  const auto rq = make_rsrc(a.q + head, n * RB);
  const auto rk = make_rsrc(a.k + head, n * RB);
  const auto rv = make_rsrc(a.v + head, n * RB);
  const Mask mk{n, a.causal, a.wl, a.wr};
  const float c = a.c;
  const float NEG_INF = -__builtin_inff();

  // transposing-read coordinates: 16-lane group g, row r of the read, half h8 of the row
  const int tgrp = lane >> 4, trow = (lane & 15) >> 1, th8 = lane & 1;
  const int tkey = 8 * (trow >> 2) + 4 * hi + (trow & 3);   // key of row r in read 0
  int vaddr[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) vaddr[db] = tile_off8<D>(tkey, 2 * db + (tgrp & 1)) + 8 * th8;
  // K operand reads: row 32 mb + l32, logical chunks 4 ks + 2 hi and 4 ks + 2 hi + 1
  int kaddr[KS][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int x = 0; x < 2; ++x) kaddr[ks][x] = tile_off8<D>(l32, 4 * ks + 2 * hi + x);

  const int npass = (a.paired && a.n_qt - 1 - unit != unit) ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
    const int qt = a.paired ? (pass == 0 ? a.n_qt - 1 - unit : unit) : unit;
    if (pass > 0) __syncthreads();   // the previous tile's last LDS reads are done

    const int q0 = qt * kBr8;
    const int wq0 = q0 + 32 * wave;
    const int wq1 = wq0 + 31;
    const int qi = wq0 + l32;

    // Q^T operands (B of S^T = K Q^T): query qi, head dims 64 ks + 32 hi .. + 31
    i32x8 qop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x0 = buffer_load16(rq, qi * RB + 64 * ks + 32 * hi);
      u32x4 x1 = buffer_load16(rq, qi * RB + 64 * ks + 32 * hi + 16);
      x0 ^= a.q_sign;
      x1 ^= a.q_sign;
      qop[ks] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                      (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    }

    int key_lo, key_hi;
    mk.key_range(q0, min(q0 + kBr8 - 1, n - 1), key_lo, key_hi);
    const int t_begin = max(key_lo, 0) / kBc8;
    const int t_end = (max(key_hi, 0) + kBc8 - 1) / kBc8;
    int wkey_lo, wkey_hi;   // keys this wave's own queries can see
    mk.key_range(wq0, min(wq1, n - 1), wkey_lo, wkey_hi);
    const bool wave_has_rows = wq0 < n;

    u32x4 kbuf[CPT], vbuf[CPT];
    auto load_tile = [&](int t) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int s = tid + kT8 * i;                  // physical 16-byte slot of the tile
        const int row = s / CPR, pch = s % CPR;
        const int src = (t * kBc8 + row) * RB + ((pch ^ swz8<D>(row)) << 4);
        kbuf[i] = buffer_load16(rk, src);
        vbuf[i] = buffer_load16(rv, src);
      }
    };
    auto store_tile = [&](int stage) __attribute__((always_inline)) {
      char FA_LDS* kt = lds + stage * 2 * TILE;
      char FA_LDS* vt = kt + TILE;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int s = tid + kT8 * i;
        lds_write16(kt, 16 * s, kbuf[i]);
        lds_write16(vt, 16 * s, vbuf[i]);
      }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m_ref = NEG_INF;   // reference exponent (base 2)
    float l_run = 0.f;       // sum of 2^(s c - m + kPS) over this lane's keys

    // One key tile.  Tiles with hidden pairs (edges, and tiles past this wave's keys) have
    // them set to -inf in a branch around the mask alone, so the accumulators see one code
    // path (no register copies where paths join); hidden scores then give P'' = 0.
    auto tile = [&](const char FA_LDS* kt, const char FA_LDS* vt, int j0, bool masked)
        __attribute__((always_inline)) {
      // ---- S^T = K Q^T: two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 k0 = lds_read16(kt, 32 * mb * RB + kaddr[ks][0]);
          const u32x4 k1 = lds_read16(kt, 32 * mb * RB + kaddr[ks][1]);
          const i32x8 kop = {(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3],
                             (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
          s[mb] = mfma_fp8(kop, qop[ks], s[mb]);
        }
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
      // ---- tile maximum; move the reference where the new maximum matters (both lanes of
      // a query see the same maximum and the same row sum, so they decide alike)
      float ext = s[0][0];
#pragma unroll
      for (int e = 1; e < 32; ++e) ext = fmaxf(ext, s[e / 16][e % 16]);
      ext = max_with_partner(ext);
      const float m_tile = __builtin_isinf(ext) ? NEG_INF : ext * c;
      const float g = m_tile - m_ref;
      const float l_row = sum_with_partner(l_run);
      const bool heavy = exp2_fast(g + 4.f + kPS) > l_row;
      const bool move = (g > 0.f) & ((g > kTau8) | heavy);
      if (__any(move)) {
        const float alpha = move ? exp2_fast(m_ref - m_tile) : 1.f;   // 0 on a first tile
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        m_ref = move ? m_tile : m_ref;
      }
      // ---- P'' = 2^(s c - m + kPS): l accumulates the unrounded values, the product takes
      // them rounded once to E4M3
      const float neg_m = (m_ref == NEG_INF ? 0.f : -m_ref) + kPS;
      float p[32];
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        // c > 0 and neg_m finite: a hidden score (-inf) gives 2^-inf = 0
        const float x = exp2_fast(__builtin_fmaf(s[e / 16][e % 16], c, neg_m));
        p[e] = x;
        part[e & 3] += x;
      }
      l_run += (part[0] + part[1]) + (part[2] + part[3]);
      i32x8 pb;
#pragma unroll
      for (int w = 0; w < 8; ++w) pb[w] = pack4_fp8(p[4 * w], p[4 * w + 1], p[4 * w + 2], p[4 * w + 3]);
      // ---- O^T += V^T P''^T
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        i32x8 vop;
#pragma unroll
        for (int rd = 0; rd < 4; ++rd) {
          const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (i32x2 FA_LDS*)(const_cast<char FA_LDS*>(vt) + 16 * rd * RB + vaddr[db]));
          vop[2 * rd] = r[0];
          vop[2 * rd + 1] = r[1];
        }
        oacc[db] = mfma_fp8(vop, pb, oacc[db]);
      }
    };

    if (t_begin < t_end) {
      load_tile(t_begin);
      store_tile(0);
    }
    __syncthreads();
    int stage = 0;
    for (int t = t_begin; t < t_end; ++t) {
      const char FA_LDS* kt = lds + stage * 2 * TILE;
      const char FA_LDS* vt = kt + TILE;
      if (t + 1 < t_end) load_tile(t + 1);
      const int j0 = t * kBc8;
      const bool live = wave_has_rows && j0 < wkey_hi && j0 + kBc8 > wkey_lo;
      tile(kt, vt, j0, !(live && mk.all_visible(wq0, wq1, j0, j0 + kBc8)));
      if (t + 1 < t_end) store_tile(stage ^ 1);
      __syncthreads();
      stage ^= 1;
    }

    // ---- epilogue: O = v_descale acc / l, LSE = ln 2 (m + log2 l - kPS)
    const float l_tot = sum_with_partner(l_run);
    if (qi < n) {
      const bool live = l_tot > 0.f;
      const float inv = live ? a.v_scale / l_tot : 0.f;
      char* orow = a.o + (long)bh * n * (2 * D) + (long)qi * (2 * D);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int dim = 32 * db + 8 * gq + 4 * hi;
          u32x2 w = {pack2<BF16OUT>(oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv),
                     pack2<BF16OUT>(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + dim * 2) = w;
        }
      if (a.lse != nullptr && hi == 0)
        a.lse[(long)bh * n + qi] = live ? (m_ref + __builtin_log2f(l_tot) - kPS) * kLn2 : NEG_INF;
    }
  }
}

template <int D, bool BF16OUT>
hipError_t launch8(const Fp8FwdParams& p, hipStream_t stream) {
  Fp8Args a;
  a.q = static_cast<const char*>(p.q);
  a.k = static_cast<const char*>(p.k);
  a.v = static_cast<const char*>(p.v);
  a.o = static_cast<char*>(p.o);
  a.lse = p.lse;
  a.n = p.N;
  a.n_bh = p.B * p.H;
  a.n_qt = (p.N + kBr8 - 1) / kBr8;
  const bool growing = p.causal && p.window_left < 0;
  a.paired = growing && (long)a.n_bh * ((a.n_qt + 1) / 2) >= 256;
  a.n_units = a.paired ? (a.n_qt + 1) / 2 : a.n_qt;
  // a zero scale becomes a tiny one: every probability is then exactly 1 (as for 0) while
  // hidden scores (-inf) still give 0
  a.c = (float)(std::fmax(std::fabs((double)p.scale) * (double)p.q_descale * (double)p.k_descale,
                          1e-30) * 1.4426950408889634);
  a.v_scale = p.v_descale;
  a.q_sign = p.scale < 0.f ? 0x80808080u : 0u;
  a.causal = p.causal;
  a.wl = p.window_left;
  a.wr = p.causal ? 0 : p.window_right;
  const long blocks = (long)a.n_bh * a.n_units;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, BF16OUT>), dim3((unsigned)blocks), dim3(kT8), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream) {
  if (p.D == 64) return p.out_bf16 ? launch8<64, true>(p, stream) : launch8<64, false>(p, stream);
  return p.out_bf16 ? launch8<128, true>(p, stream) : launch8<128, false>(p, stream);
}

}  // namespace fa
