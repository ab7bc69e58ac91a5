// Attention backward for gfx950, by recomputation.
//
// Nothing of the forward's N x N intermediates was kept; only O and the per-query
// logsumexp LSE.  The probabilities are rebuilt tile by tile as P = exp(S*scale - LSE),
// which is the recomputation named by "PyTorch-CUDA-v2.9镜像中使用FlashAttention提升训练速度"
// ("3. 重计算策略（Recomputation）") and by "告别OOM和训练慢：用Flash Attention加速你的PyTorch大模型
// （含A100环境配置）" §2.2 (only the normalisation statistics are kept for the backward pass).
// The gradients are the ordinary derivative of softmax(scale Q K^T + mask) V:
//
//     dV = P^T dO      dP = dO V^T      dS = P * (dP - delta),  delta_i = sum_c dO_ic O_ic
//     dK = scale dS^T Q                  dQ = scale dS K
//
// Three kernels, all deterministic (no atomics):
//   delta_kernel  delta = rowsum(dO * O) in fp32                      (bandwidth bound)
//   dkdv_kernel   one workgroup per 128 keys; loops over the query tiles that can see them:
//                 S = Q K^T and dP = dO V^T with K^T, V^T held in registers, then
//                 dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T read transposed from LDS
//   dq_kernel     one workgroup per 128 queries; loops over the visible key tiles:
//                 S^T = K Q^T and dP^T = V dO^T with Q^T, dO^T in registers, then
//                 dQ^T += K^T dS^T with K^T read transposed from LDS
// Each score tile is laid out so that the accumulator registers of S / dP are directly the
// MFMA operand that P / dS feed, as in the forward kernel.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "cdna4.h"
#include "launch.h"

namespace fa {

namespace {

struct BwdArgs {
  const char* q;
  const char* k;
  const char* v;
  const char* o;
  const char* dout;
  const float* lse;
  char* dq;
  char* dk;
  char* dv;
  float* stats;   // per-query statistics in 32-query blocks (stat_index)
  const int* seqlens;   // per-batch lengths (device, may be null); only the delta pass reads them
  int heads;
  int n;
  int n_bh;
  int n_tiles;
  float c;        // sigma * log2(e)
  float sigma;    // softmax_scale kept away from zero (softmax_sigma)
  float scale;    // softmax_scale
  int causal, wl, wr;
};

// ---------------------------------------------------------------------------- delta
// delta = sum_c dO[c] * O[c] per query with both rounded inputs in fp32, stored negated next
// to m = -LSE / sigma (the exponent offset the recomputation of P needs); slots of the padded
// statistics blocks past the sequence get zeros.  A row is D / 8 lanes of 16 bytes, so every
// load instruction of a wave reads 64 / (D / 8) whole consecutive rows (1 KiB, no partial
// lines); the lanes of a row add their partial sums by butterfly shuffles.
// Grid: x over a head's padded query slots, 256 per workgroup (64 per wave); y, with a stride
// loop, over (batch, head).
// PADDED: a padded batch (per-batch lengths), a separate instance
template <int D, bool BF16, bool PADDED>
__global__ __launch_bounds__(256) void delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;            // lanes per row
  constexpr int RPI = 64 / LPR;         // rows per load instruction
  constexpr int IT = 64 / RPI;          // load instructions per wave and tensor
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR;
  const int q_base = blockIdx.x * 256 + (threadIdx.x >> 6) * 64 + lane / LPR;
  const int slots = stat_blocks(a.n) * kStatRows;
  for (long bh = blockIdx.y; bh < a.n_bh; bh += gridDim.y) {
    // rows of the sequence; rows len .. n-1 of a padded batch get zeros like the slots past n
    const int len = PADDED ? min(max(a.seqlens[bh / a.heads], 0), a.n) : a.n;
    u32x4 ov[IT], gv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int q = q_base + RPI * it;
      ov[it] = gv[it] = u32x4{};
      if (q < len) {
        const long off = ((bh * a.n + q) * D + 8 * sub) * 2;
        ov[it] = *reinterpret_cast<const u32x4*>(a.o + off);
        gv[it] = *reinterpret_cast<const u32x4*>(a.dout + off);
      }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc += to_float<BF16>((unsigned short)(ov[it][w] & 0xffff)) *
               to_float<BF16>((unsigned short)(gv[it][w] & 0xffff));
        acc += to_float<BF16>((unsigned short)(ov[it][w] >> 16)) *
               to_float<BF16>((unsigned short)(gv[it][w] >> 16));
      }
#pragma unroll
      for (int x = 1; x < LPR; x *= 2) acc += __shfl_xor(acc, x);
      const int q = q_base + RPI * it;
      if (sub == 0 && q < slots) {
        float* out = a.stats + stat_index(bh, a.n, q);
        const bool in = q < len;
        out[0] = in ? -a.lse[bh * a.n + q] / a.sigma : 0.f;
        out[kStatRows] = in ? -acc : 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------- dK, dV
constexpr int kKvRows = 128;   // keys per workgroup (32 per wave)
constexpr int kQStep = 32;     // queries per step

template <int D, bool BF16>
__global__ __launch_bounds__(256) void dkdv_kernel(BwdArgs a) {
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kQStep * kRowBytes;    // one Q or dO tile
  constexpr int kChunks = D / 8;
  constexpr int kLoads = kQStep * kChunks / 256;     // 16-byte chunks per thread per tile
  constexpr int kKs = D / 16;
  constexpr int kDb = D / 32;
  constexpr int kStage = 2 * kTileBytes + 2 * kQStep * 4;

  __shared__ __attribute__((aligned(16))) char lds_raw[2 * kStage];
  char FA_LDS* lds = (char FA_LDS*)(lds_raw);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  int bh, kt;
  xcd_tile_order(blockIdx.x, a.n_bh, a.n_tiles, bh, kt);
  const int n = a.n;
  const long head = (long)bh * n * kRowBytes;
  const int head_bytes = n * kRowBytes;
  const auto rq = make_rsrc(a.q + head, head_bytes);
  const auto rk = make_rsrc(a.k + head, head_bytes);
  const auto rv = make_rsrc(a.v + head, head_bytes);
  const auto rg = make_rsrc(a.dout + head, head_bytes);

  // K^T and V^T as B operands: lane holds key (k0 + l32), head-dim chunk 2 ks + hi.
  const int k_first = kt * kKvRows;
  const int key = k_first + 32 * wave + l32;
  i16x8 kreg[kKs], vreg[kKs];
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks) {
    kreg[ks] = __builtin_bit_cast(i16x8, buffer_load16(rk, key * kRowBytes + (2 * ks + hi) * 16));
    vreg[ks] = __builtin_bit_cast(i16x8, buffer_load16(rv, key * kRowBytes + (2 * ks + hi) * 16));
  }

  const Mask mk{n, a.causal, a.wl, a.wr};
  const int k_last = min(k_first + kKvRows, n) - 1;
  int q_lo, q_hi;
  mk.query_range(k_first, k_last, q_lo, q_hi);
  const int s_begin = q_lo / kQStep;
  const int s_end = q_hi > q_lo ? (q_hi + kQStep - 1) / kQStep : s_begin;

  u32x4 qbuf[kLoads], gbuf[kLoads];
  float lse_buf = 0.f, delta_buf = 0.f;   // row statistics, threads tid < kQStep
  auto load_tile = [&](int s) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + 256 * i;
      const int off = (s * kQStep + c / kChunks) * kRowBytes + (c % kChunks) * 16;
      qbuf[i] = buffer_load16(rq, off);
      gbuf[i] = buffer_load16(rg, off);
    }
    const int q = s * kQStep + tid;
    if (tid < kQStep && q < n) {
      lse_buf = a.stats[stat_index(bh, n, q)];
      delta_buf = a.stats[stat_index(bh, n, q) + kStatRows];
    } else {
      lse_buf = 0.f;
      delta_buf = 0.f;
    }
  };
  auto store_tile = [&](int stage) {
    char FA_LDS* base = lds + stage * kStage;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + 256 * i;
      const int off = tile_offset<D>(c / kChunks, c % kChunks);
      lds_write16(base, off, qbuf[i]);
      lds_write16(base + kTileBytes, off, gbuf[i]);
    }
    if (tid < kQStep) {
      float FA_LDS* st = (float FA_LDS*)(base + 2 * kTileBytes);
      st[tid] = lse_buf;
      st[kQStep + tid] = delta_buf;
    }
  };

  f32x16 dk[kDb], dv[kDb];
#pragma unroll
  for (int db = 0; db < kDb; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  const float c = a.c;

  if (s_begin < s_end) {
    load_tile(s_begin);
    store_tile(0);
  }
  __syncthreads();

  const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
  const int tr_row = (tg >> 1) * 4 + tr;
  const int tr_byte = (tq & 1) * 8;

  for (int s = s_begin; s < s_end; ++s) {
    const int stage = (s - s_begin) & 1;
    const char FA_LDS* qt = lds + stage * kStage;
    const char FA_LDS* gt = qt + kTileBytes;
    const float FA_LDS* st_lse = (const float FA_LDS*)(qt + 2 * kTileBytes);
    const float FA_LDS* st_delta = st_lse + kQStep;
    if (s + 1 < s_end) load_tile(s + 1);

    // S = Q K^T and dP = dO V^T: C[m = query][n = key], 32 queries x this wave's 32 keys
    f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      const int off = tile_offset<D>(l32, 2 * ks + hi);
      sc = mfma32x32x16<BF16>(__builtin_bit_cast(i16x8, lds_read16(qt, off)), kreg[ks], sc);
      dp = mfma32x32x16<BF16>(__builtin_bit_cast(i16x8, lds_read16(gt, off)), vreg[ks], dp);
    }

    const int q0 = s * kQStep;
    const bool full = mk.all_visible(q0, q0 + kQStep - 1, k_first, k_first + kKvRows) &&
                      q0 + kQStep <= n;
    unsigned pk[8], dk_pk[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // queries 8 g + 4 hi + 0..3 of this step
      const f32x4 l2 = *reinterpret_cast<const f32x4 FA_LDS*>(st_lse + 8 * g + 4 * hi);
      const f32x4 de = *reinterpret_cast<const f32x4 FA_LDS*>(st_delta + 8 * g + 4 * hi);
      float p[4], d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * g + e;
        float pe = exp2_fast(__builtin_fmaf(sc[i], c, c * l2[e]));
        if (!full) {
          const int qq = q0 + 8 * g + 4 * hi + e;
          pe = (qq < n && mk.visible(qq, key)) ? pe : 0.f;
        }
        p[e] = pe;
        d[e] = pe * (dp[i] + de[e]);
      }
      pk[2 * g] = pack2<BF16>(p[0], p[1]);
      pk[2 * g + 1] = pack2<BF16>(p[2], p[3]);
      dk_pk[2 * g] = pack2<BF16>(d[0], d[1]);
      dk_pk[2 * g + 1] = pack2<BF16>(d[2], d[3]);
    }

    // dV^T += dO^T P and dK^T += Q^T dS: C[m = head dim][n = key], contraction over queries
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 pb = {pk[4 * kk], pk[4 * kk + 1], pk[4 * kk + 2], pk[4 * kk + 3]};
      const u32x4 sb = {dk_pk[4 * kk], dk_pk[4 * kk + 1], dk_pk[4 * kk + 2], dk_pk[4 * kk + 3]};
      const int row = 16 * kk + tr_row;
#pragma unroll
      for (int db = 0; db < kDb; ++db) {
        const int chunk = 4 * db + 2 * (tg & 1) + (tq >> 1);
        const int off_a = tile_offset<D>(row, chunk) + tr_byte;
        const int off_b = tile_offset<D>(row + 8, chunk) + tr_byte;
        const i16x8 go = __builtin_shufflevector(lds_read_tr(gt, off_a), lds_read_tr(gt, off_b),
                                                 0, 1, 2, 3, 4, 5, 6, 7);
        const i16x8 qo = __builtin_shufflevector(lds_read_tr(qt, off_a), lds_read_tr(qt, off_b),
                                                 0, 1, 2, 3, 4, 5, 6, 7);
        dv[db] = mfma32x32x16<BF16>(go, __builtin_bit_cast(i16x8, pb), dv[db]);
        dk[db] = mfma32x32x16<BF16>(qo, __builtin_bit_cast(i16x8, sb), dk[db]);
      }
    }

    if (s + 1 < s_end) store_tile(stage ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds key (k_first + 32 wave + l32), dims 32 db + 8 g + 4 hi + 0..3
  if (key < n) {
    char* dkrow = a.dk + head + (long)key * kRowBytes;
    char* dvrow = a.dv + head + (long)key * kRowBytes;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < kDb; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = 32 * db + 8 * g + 4 * hi;
        u32x2 wk = {pack2<BF16>(dk[db][4 * g + 0] * sc, dk[db][4 * g + 1] * sc),
                    pack2<BF16>(dk[db][4 * g + 2] * sc, dk[db][4 * g + 3] * sc)};
        u32x2 wv = {pack2<BF16>(dv[db][4 * g + 0], dv[db][4 * g + 1]),
                    pack2<BF16>(dv[db][4 * g + 2], dv[db][4 * g + 3])};
        *reinterpret_cast<u32x2*>(dkrow + dim * 2) = wk;
        *reinterpret_cast<u32x2*>(dvrow + dim * 2) = wv;
      }
  }
}

// ---------------------------------------------------------------------------- dQ
constexpr int kDqRows = 128;   // queries per workgroup (32 per wave)
constexpr int kKStep = 64;     // keys per K/V tile

template <int D, bool BF16>
__global__ __launch_bounds__(256) void dq_kernel(BwdArgs a) {
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kKStep * kRowBytes;
  constexpr int kChunks = D / 8;
  constexpr int kLoads = kKStep * kChunks / 256;
  constexpr int kKs = D / 16;
  constexpr int kDb = D / 32;

  __shared__ __attribute__((aligned(16))) char lds_raw[2 * 2 * kTileBytes];
  char FA_LDS* lds = (char FA_LDS*)(lds_raw);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  int bh, qt;
  xcd_tile_order(blockIdx.x, a.n_bh, a.n_tiles, bh, qt);
  if (a.causal) qt = a.n_tiles - 1 - qt;
  const int n = a.n;
  const int q0 = qt * kDqRows;
  const long head = (long)bh * n * kRowBytes;
  const int head_bytes = n * kRowBytes;
  const auto rq = make_rsrc(a.q + head, head_bytes);
  const auto rk = make_rsrc(a.k + head, head_bytes);
  const auto rv = make_rsrc(a.v + head, head_bytes);
  const auto rg = make_rsrc(a.dout + head, head_bytes);

  const int qi = q0 + 32 * wave + l32;
  i16x8 qreg[kKs], greg[kKs];
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks) {
    qreg[ks] = __builtin_bit_cast(i16x8, buffer_load16(rq, qi * kRowBytes + (2 * ks + hi) * 16));
    greg[ks] = __builtin_bit_cast(i16x8, buffer_load16(rg, qi * kRowBytes + (2 * ks + hi) * 16));
  }
  const bool row_ok = qi < n;
  const float mrow = row_ok ? a.stats[stat_index(bh, n, qi)] : 0.f;               // -LSE / sigma
  const float ndlt = row_ok ? a.stats[stat_index(bh, n, qi) + kStatRows] : 0.f;   // -delta

  const Mask mk{n, a.causal, a.wl, a.wr};
  const int q_last = q0 + kDqRows - 1;
  int key_lo, key_hi;
  mk.key_range(q0, min(q_last, n - 1), key_lo, key_hi);
  const int t_begin = key_lo / kKStep;
  const int t_end = (key_hi + kKStep - 1) / kKStep;

  u32x4 kbuf[kLoads], vbuf[kLoads];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int cc = tid + 256 * i;
      const int off = (t * kKStep + cc / kChunks) * kRowBytes + (cc % kChunks) * 16;
      kbuf[i] = buffer_load16(rk, off);
      vbuf[i] = buffer_load16(rv, off);
    }
  };
  auto store_tile = [&](int stage) {
    char FA_LDS* kt = lds + stage * 2 * kTileBytes;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int cc = tid + 256 * i;
      const int off = tile_offset<D>(cc / kChunks, cc % kChunks);
      lds_write16(kt, off, kbuf[i]);
      lds_write16(kt + kTileBytes, off, vbuf[i]);
    }
  };

  f32x16 dqacc[kDb];
#pragma unroll
  for (int db = 0; db < kDb; ++db) dqacc[db] = f32x16{};
  const float c = a.c;
  const float cm = c * mrow;   // -log2(e) LSE

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
  }
  __syncthreads();

  const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
  const int tr_key = (tg >> 1) * 4 + tr;
  const int tr_byte = (tq & 1) * 8;

  for (int t = t_begin; t < t_end; ++t) {
    const int stage = (t - t_begin) & 1;
    const char FA_LDS* kt = lds + stage * 2 * kTileBytes;
    const char FA_LDS* vt = kt + kTileBytes;
    if (t + 1 < t_end) load_tile(t + 1);

    // S^T = K Q^T and dP^T = V dO^T: C[m = key][n = query]
    f32x16 sc[2], dp[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sc[mb] = f32x16{};
      dp[mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        const int off = tile_offset<D>(32 * mb + l32, 2 * ks + hi);
        sc[mb] = mfma32x32x16<BF16>(__builtin_bit_cast(i16x8, lds_read16(kt, off)), qreg[ks], sc[mb]);
        dp[mb] = mfma32x32x16<BF16>(__builtin_bit_cast(i16x8, lds_read16(vt, off)), greg[ks], dp[mb]);
      }
    }

    const int j0 = t * kKStep;
    const bool full = mk.all_visible(q0, q_last, j0, j0 + kKStep);
    unsigned dsk[2][8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float d2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float p = exp2_fast(__builtin_fmaf(sc[mb][i + e], c, cm));
          if (!full) {
            const int j = j0 + 32 * mb + 8 * ((i + e) >> 2) + 4 * hi + ((i + e) & 3);
            p = (row_ok && mk.visible(qi, j)) ? p : 0.f;
          }
          d2[e] = p * (dp[mb][i + e] + ndlt);
        }
        dsk[mb][i >> 1] = pack2<BF16>(d2[0], d2[1]);
      }

    // dQ^T += K^T dS^T: C[m = head dim][n = query], contraction over keys
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 sb = {dsk[kk >> 1][4 * (kk & 1) + 0], dsk[kk >> 1][4 * (kk & 1) + 1],
                        dsk[kk >> 1][4 * (kk & 1) + 2], dsk[kk >> 1][4 * (kk & 1) + 3]};
      const int key_a = 16 * kk + tr_key;
#pragma unroll
      for (int db = 0; db < kDb; ++db) {
        const int chunk = 4 * db + 2 * (tg & 1) + (tq >> 1);
        const i16x8 ko = __builtin_shufflevector(
            lds_read_tr(kt, tile_offset<D>(key_a, chunk) + tr_byte),
            lds_read_tr(kt, tile_offset<D>(key_a + 8, chunk) + tr_byte), 0, 1, 2, 3, 4, 5, 6, 7);
        dqacc[db] = mfma32x32x16<BF16>(ko, __builtin_bit_cast(i16x8, sb), dqacc[db]);
      }
    }

    if (t + 1 < t_end) store_tile(stage ^ 1);
    __syncthreads();
  }

  if (row_ok) {
    char* row = a.dq + head + (long)qi * kRowBytes;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < kDb; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = 32 * db + 8 * g + 4 * hi;
        u32x2 w = {pack2<BF16>(dqacc[db][4 * g + 0] * sc, dqacc[db][4 * g + 1] * sc),
                   pack2<BF16>(dqacc[db][4 * g + 2] * sc, dqacc[db][4 * g + 3] * sc)};
        *reinterpret_cast<u32x2*>(row + dim * 2) = w;
      }
  }
}

// Backward kernel requested through the environment (FA_BWD_KERNEL = "main" or "basic"),
// 0 if unset.  A tuning and testing knob, read at every call and ignored unless set.
int env_bwd_choice() {
  const char* e = std::getenv("FA_BWD_KERNEL");
  if (e == nullptr) return 0;
  if (std::strcmp(e, "main") == 0) return 1;
  if (std::strcmp(e, "basic") == 0) return 2;
  return 0;
}

BwdArgs make_args(const BwdParams& p) {
  BwdArgs a;
  a.q = static_cast<const char*>(p.q);
  a.k = static_cast<const char*>(p.k);
  a.v = static_cast<const char*>(p.v);
  a.o = static_cast<const char*>(p.o);
  a.dout = static_cast<const char*>(p.dout);
  a.lse = p.lse;
  a.dq = static_cast<char*>(p.dq);
  a.dk = static_cast<char*>(p.dk);
  a.dv = static_cast<char*>(p.dv);
  a.stats = p.stats;
  a.seqlens = p.seqlens;
  a.heads = p.H;
  a.n = p.N;
  a.n_bh = p.B * p.H;
  a.n_tiles = 0;
  a.sigma = softmax_sigma(p.scale);
  a.c = (float)((double)a.sigma * 1.4426950408889634);
  a.scale = p.scale;
  a.causal = p.causal;
  a.wl = p.window_left;
  a.wr = p.causal ? 0 : p.window_right;   // causal is a right bound of 0
  return a;
}

template <int D, bool BF16>
hipError_t launch(const BwdParams& p, unsigned stages, hipStream_t stream) {
  BwdArgs a = make_args(p);
  if (stages & kBwdDelta) {
    const unsigned gx = (unsigned)((stat_blocks(a.n) * kStatRows + 255) / 256);
    const unsigned gy = (unsigned)std::min(a.n_bh, 65535);
    if (p.seqlens != nullptr)
      hipLaunchKernelGGL((delta_kernel<D, BF16, true>), dim3(gx, gy), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((delta_kernel<D, BF16, false>), dim3(gx, gy), dim3(256), 0, stream, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  // padded batches always take the main kernels
  const bool main_kernels = env_bwd_choice() != 2 || p.seqlens != nullptr;
  if ((stages & kBwdDkDv) && main_kernels) {
    if (hipError_t e = launch_dkdv_main(p, stream); e != hipSuccess) return e;
  } else if (stages & kBwdDkDv) {
    a.n_tiles = (a.n + kKvRows - 1) / kKvRows;
    hipLaunchKernelGGL((dkdv_kernel<D, BF16>), dim3((unsigned)((long)a.n_bh * a.n_tiles)), dim3(256),
                       0, stream, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  if ((stages & kBwdDq) && main_kernels) {
    if (hipError_t e = launch_dq_main(p, stream); e != hipSuccess) return e;
  } else if (stages & kBwdDq) {
    a.n_tiles = (a.n + kDqRows - 1) / kDqRows;
    hipLaunchKernelGGL((dq_kernel<D, BF16>), dim3((unsigned)((long)a.n_bh * a.n_tiles)), dim3(256), 0,
                       stream, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, unsigned stages, hipStream_t stream) {
  if (p.D == 64) return p.bf16 ? launch<64, true>(p, stages, stream) : launch<64, false>(p, stages, stream);
  return p.bf16 ? launch<128, true>(p, stages, stream) : launch<128, false>(p, stages, stream);
}

}  // namespace fa
