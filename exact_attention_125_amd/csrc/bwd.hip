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
  const int* cu;        // packed batch: per-batch start rows [B + 1] (device), or null
  int total;            // packed batch: rows per head
  const float* slopes;  // ALiBi slopes [heads] (device), read by the ALIBI instances only
  Dropout drop;         // used by the DROPOUT instances only
  const unsigned char* blocks;   // block-sparse mask [heads][n_qb][n_kb] of 64 x 64 blocks, or null
  const unsigned char* kpm;      // key padding mask [batch][nk] (nonzero = padding key), or null
  int n_qb, n_kb;
  // batch / head strides (bytes) and row strides (bytes) of q, k, v, o, dout, dq, dk, dv
  long long q_bs, q_hs, k_bs, k_hs, v_bs, v_hs, o_bs, o_hs, g_bs, g_hs;
  long long dq_bs, dq_hs, dk_bs, dk_hs, dv_bs, dv_hs;
  int q_rs, k_rs, v_rs, o_rs, g_rs, dq_rs, dk_rs, dv_rs;
  int heads;
  int n;          // query rows (statistics, LSE)
  int nk;         // key rows
  int off;        // key position of query 0 (nk - n)
  int n_bh;
  int n_tiles;
  float c;        // sigma * log2(e)
  float sigma;    // softmax_scale kept away from zero (softmax_sigma)
  float scale;    // softmax_scale
  int causal, wl, wr;
};

// Buffer resource over rows [0, rows) with a row stride of rs bytes (rows at or past the end
// read as zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const char* base, int rows, int rs,
                                                            int row_bytes) {
  return make_rsrc(base, rows > 0 ? (rows - 1) * rs + row_bytes : 0);
}

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
    // (a packed batch: sequence b is rows cu[b] .. cu[b+1]-1 of each head's `total` rows,
    // offsets clamped to [0, total], at most n rows)
    const int b = (int)(bh / a.heads), h = (int)(bh - (long)b * a.heads);
    int len = a.n;
    long row0 = 0, lrow = bh * a.n;
    if constexpr (PADDED) {
      if (a.cu != nullptr) {
        const int c0 = min(max(a.cu[b], 0), a.total);
        const int c1 = min(max(a.cu[b + 1], c0), a.total);
        len = min(c1 - c0, a.n);
        row0 = c0;
        lrow = (long)h * a.total + c0;
      } else {
        len = min(max(a.seqlens[b], 0), a.n);
      }
    }
    const char* orows = a.o + b * a.o_bs + h * a.o_hs + row0 * a.o_rs + 16 * sub;
    const char* grows = a.dout + b * a.g_bs + h * a.g_hs + row0 * a.g_rs + 16 * sub;
    u32x4 ov[IT], gv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int q = q_base + RPI * it;
      ov[it] = gv[it] = u32x4{};
      if (q < len) {
        ov[it] = *reinterpret_cast<const u32x4*>(orows + (long)q * a.o_rs);
        gv[it] = *reinterpret_cast<const u32x4*>(grows + (long)q * a.g_rs);
      }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float acc = delta_chunk<BF16>(ov[it], gv[it]);
      // lanes of a row exchange sums at distance 1, 2, 4 ...: the pairwise order of delta_chunk
#pragma unroll
      for (int x = 1; x < LPR; x *= 2) acc += __shfl_xor(acc, x);
      const int q = q_base + RPI * it;
      if (sub == 0 && q < slots) {
        float* out = a.stats + stat_index(bh, a.n, q);
        const bool in = q < len;
        // a row that sees no key (LSE = -inf; only with fewer keys than queries or a window)
        // gets zeros too: every one of its scores is masked
        const float lse = in ? a.lse[lrow + q] : 0.f;
        const bool live = in && lse != -__builtin_inff();
        out[0] = live ? -lse / a.sigma : 0.f;
        out[kStatRows] = live ? -acc : 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------- dK, dV
constexpr int kKvRows = 128;   // keys per workgroup (32 per wave)
constexpr int kQStep = 32;     // queries per step

// ALIBI: P carries the forward's ALiBi penalty, 2^(... - slope log2(e) |p - j|).
// DROPOUT: the forward's weights were P * keep * s (s = a.drop.scale, the inverse of the keep
// probability), so dV uses them and dP is (dO V^T) * keep * s, with keep drawn again from
// a.drop.
template <int D, bool BF16, bool ALIBI, bool DROPOUT>
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
  const int n = a.n, nk = a.nk, off = a.off;   // queries, keys, key position of query 0
  const int b = bh / a.heads, h = bh - b * a.heads;
  const auto rq = rows_rsrc(a.q + b * a.q_bs + h * a.q_hs, n, a.q_rs, kRowBytes);
  const auto rk = rows_rsrc(a.k + b * a.k_bs + h * a.k_hs, nk, a.k_rs, kRowBytes);
  const auto rv = rows_rsrc(a.v + b * a.v_bs + h * a.v_hs, nk, a.v_rs, kRowBytes);
  const auto rg = rows_rsrc(a.dout + b * a.g_bs + h * a.g_hs, n, a.g_rs, kRowBytes);
  const float b2 = ALIBI ? a.slopes[h] * kLog2e : 0.f;

  // K^T and V^T as B operands: lane holds key (k0 + l32), head-dim chunk 2 ks + hi.
  const int k_first = kt * kKvRows;
  const int key = k_first + 32 * wave + l32;
  i16x8 kreg[kKs], vreg[kKs];
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks) {
    kreg[ks] = __builtin_bit_cast(i16x8, buffer_load16(rk, key * a.k_rs + (2 * ks + hi) * 16));
    vreg[ks] = __builtin_bit_cast(i16x8, buffer_load16(rv, key * a.v_rs + (2 * ks + hi) * 16));
  }
  // key padding: this lane's key is hidden from every query (its dK and dV stay zero); a wave
  // whose keys are all padding (or past the last key) computes nothing
  const bool kpad = a.kpm != nullptr && key < nk && a.kpm[(long)b * nk + key] != 0;
  const bool wave_idle = a.kpm != nullptr && __all(kpad || key >= nk);

  // queries that see any of the keys: the mask works on positions (index + off), which
  // start at off (negative when there are more queries than keys)
  const Mask mk{nk, a.causal, a.wl, a.wr};
  const int k_last = min(k_first + kKvRows, nk) - 1;
  int p_lo = off, p_hi = off + n;                        // positions [p_lo, p_hi)
  if (a.causal) p_lo = max(p_lo, k_first);
  if (a.wr >= 0) p_lo = max(p_lo, k_first - a.wr);
  if (a.wl >= 0) p_hi = min(p_hi, k_last + a.wl + 1);
  const int q_lo = max(p_lo - off, 0), q_hi = min(p_hi - off, n);
  const int s_begin = q_lo / kQStep;
  const int s_end = q_hi > q_lo ? (q_hi + kQStep - 1) / kQStep : s_begin;

  u32x4 qbuf[kLoads], gbuf[kLoads];
  float lse_buf = 0.f, delta_buf = 0.f;   // row statistics, threads tid < kQStep
  auto load_tile = [&](int s) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + 256 * i;
      const int row = s * kQStep + c / kChunks, col = (c % kChunks) * 16;
      qbuf[i] = buffer_load16(rq, row * a.q_rs + col);
      gbuf[i] = buffer_load16(rg, row * a.g_rs + col);
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

  // Block-sparse: the workgroup visits only the query steps that one of its two 64-key block
  // columns selects (the others are neither loaded nor waited for).
  const int kb0 = k_first / 64, kb1 = min(kb0 + 1, a.n_kb - 1);
  auto next_step = [&](int s) {   // first visited step at or after s (32 queries = half a block)
    if (a.blocks != nullptr) {
      const unsigned char* hm = a.blocks + (long)h * a.n_qb * a.n_kb;
      while (s < s_end && !(hm[(s >> 1) * a.n_kb + kb0] | hm[(s >> 1) * a.n_kb + kb1])) ++s;
    }
    return s;
  };
  const int s_first = next_step(s_begin);
  if (s_first < s_end) {
    load_tile(s_first);
    store_tile(0);
  }
  __syncthreads();

  const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
  const int tr_row = (tg >> 1) * 4 + tr;
  const int tr_byte = (tq & 1) * 8;

  int stage = 0;
  for (int s = s_first; s < s_end;) {
    const char FA_LDS* qt = lds + stage * kStage;
    const char FA_LDS* gt = qt + kTileBytes;
    const float FA_LDS* st_lse = (const float FA_LDS*)(qt + 2 * kTileBytes);
    const float FA_LDS* st_delta = st_lse + kQStep;
    const int s_next = next_step(s + 1);
    if (s_next < s_end) load_tile(s_next);

    // block-sparse: this wave's 32 keys and the step's 32 queries lie in one 64 x 64 block;
    // an unselected block contributes nothing (the wave still takes part in the copies)
    // (a wave past the last key has no output: it skips, and reads no mask entry)
    if (!wave_idle &&
        (a.blocks == nullptr ||
         (k_first + 32 * wave < nk &&
          a.blocks[((long)h * a.n_qb + (s * kQStep) / 64) * a.n_kb + (k_first + 32 * wave) / 64]))) {
    // S = Q K^T and dP = dO V^T: C[m = query][n = key], 32 queries x this wave's 32 keys
    f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      const int off = tile_offset<D>(l32, 2 * ks + hi);
      sc = mfma32x32x16<BF16>(__builtin_bit_cast(i16x8, lds_read16(qt, off)), kreg[ks], sc);
      dp = mfma32x32x16<BF16>(__builtin_bit_cast(i16x8, lds_read16(gt, off)), vreg[ks], dp);
    }

    const int q0 = s * kQStep;
    const bool full = mk.all_visible(q0 + off, q0 + kQStep - 1 + off, k_first, k_first + kKvRows) &&
                      q0 + kQStep <= n;
    unsigned pk[8], dk_pk[8];
    // DROPOUT: this key's draws for the step's query pairs 8 g + 4 hi + 2 c' + {0, 1}
    unsigned rw[8][2];
    if constexpr (DROPOUT) a.drop.pairs8(bh, q0 + 4 * hi, key, rw);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // queries 8 g + 4 hi + 0..3 of this step
      const f32x4 l2 = *reinterpret_cast<const f32x4 FA_LDS*>(st_lse + 8 * g + 4 * hi);
      const f32x4 de = *reinterpret_cast<const f32x4 FA_LDS*>(st_delta + 8 * g + 4 * hi);
      float p[4], d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * g + e;
        float x = __builtin_fmaf(sc[i], c, c * l2[e]);
        if constexpr (ALIBI)
          x = __builtin_fmaf(-b2, __builtin_fabsf((float)(q0 + 8 * g + 4 * hi + e + off - key)), x);
        float pe = exp2_fast(x);
        if (!full) {
          const int qq = q0 + 8 * g + 4 * hi + e;
          pe = (qq < n && mk.visible(qq + off, key)) ? pe : 0.f;
        }
        pe = kpad ? 0.f : pe;
        if constexpr (DROPOUT) {
          const bool kept = a.drop.keep_half(rw[2 * g + (e >> 1)][e & 1], key & 1);
          p[e] = kept ? pe * a.drop.scale : 0.f;
          d[e] = pe * ((kept ? dp[i] * a.drop.scale : 0.f) + de[e]);
        } else {
          p[e] = pe;
          d[e] = pe * (dp[i] + de[e]);
        }
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
    }   // selected block

    if (s_next < s_end) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    s = s_next;
  }

  // epilogue: lane holds key (k_first + 32 wave + l32), dims 32 db + 8 g + 4 hi + 0..3
  if (key < nk) {
    char* dkrow = a.dk + b * a.dk_bs + h * a.dk_hs + (long)key * a.dk_rs;
    char* dvrow = a.dv + b * a.dv_bs + h * a.dv_hs + (long)key * a.dv_rs;
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

template <int D, bool BF16, bool ALIBI, bool DROPOUT>
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
  const int n = a.n, nk = a.nk, off = a.off;   // queries, keys, key position of query 0
  const int q0 = qt * kDqRows;
  const int b = bh / a.heads, h = bh - b * a.heads;
  const auto rq = rows_rsrc(a.q + b * a.q_bs + h * a.q_hs, n, a.q_rs, kRowBytes);
  const auto rk = rows_rsrc(a.k + b * a.k_bs + h * a.k_hs, nk, a.k_rs, kRowBytes);
  const auto rv = rows_rsrc(a.v + b * a.v_bs + h * a.v_hs, nk, a.v_rs, kRowBytes);
  const auto rg = rows_rsrc(a.dout + b * a.g_bs + h * a.g_hs, n, a.g_rs, kRowBytes);
  const float b2 = ALIBI ? a.slopes[h] * kLog2e : 0.f;

  const int qi = q0 + 32 * wave + l32;
  i16x8 qreg[kKs], greg[kKs];
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks) {
    qreg[ks] = __builtin_bit_cast(i16x8, buffer_load16(rq, qi * a.q_rs + (2 * ks + hi) * 16));
    greg[ks] = __builtin_bit_cast(i16x8, buffer_load16(rg, qi * a.g_rs + (2 * ks + hi) * 16));
  }
  const bool row_ok = qi < n;
  const float mrow = row_ok ? a.stats[stat_index(bh, n, qi)] : 0.f;               // -LSE / sigma
  const float ndlt = row_ok ? a.stats[stat_index(bh, n, qi) + kStatRows] : 0.f;   // -delta

  const Mask mk{nk, a.causal, a.wl, a.wr};
  const int q_last = q0 + kDqRows - 1;
  int key_lo, key_hi;
  mk.key_range(q0 + off, min(q_last, n - 1) + off, key_lo, key_hi);
  const int t_begin = max(key_lo, 0) / kKStep;
  const int t_end = (max(key_hi, 0) + kKStep - 1) / kKStep;

  u32x4 kbuf[kLoads], vbuf[kLoads];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int cc = tid + 256 * i;
      const int row = t * kKStep + cc / kChunks, col = (cc % kChunks) * 16;
      kbuf[i] = buffer_load16(rk, row * a.k_rs + col);
      vbuf[i] = buffer_load16(rv, row * a.v_rs + col);
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
  // key padding: this batch entry's row of the mask
  const unsigned char* kpm = a.kpm ? a.kpm + (long)b * nk : nullptr;

  // Block-sparse: the workgroup visits only the key tiles that one of its two 64-query block
  // rows selects.
  const unsigned char* wg_row0 =
      a.blocks ? a.blocks + ((long)h * a.n_qb + q0 / 64) * a.n_kb : nullptr;
  const unsigned char* wg_row1 =
      (a.blocks && q0 / 64 + 1 < a.n_qb) ? wg_row0 + a.n_kb : wg_row0;
  auto next_tile = [&](int t) {
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

  const int tg = lane >> 4, tr = (lane >> 2) & 3, tq = lane & 3;
  const int tr_key = (tg >> 1) * 4 + tr;
  const int tr_byte = (tq & 1) * 8;

  int stage = 0;
  for (int t = t_first; t < t_end;) {
    const char FA_LDS* kt = lds + stage * 2 * kTileBytes;
    const char FA_LDS* vt = kt + kTileBytes;
    const int t_next = next_tile(t + 1);
    if (t_next < t_end) load_tile(t_next);

    // key padding: bit i of pad marks key t * kKStep + i as padding (keys past nk count as
    // padding here; the sequence mask hides them anyway)
    unsigned long long pad = 0;
    if (kpm != nullptr) pad = __ballot(t * kKStep + lane >= nk || kpm[t * kKStep + lane] != 0);
    // block-sparse: this wave's 32 queries and the 64-key tile lie in one 64 x 64 block
    // (a wave past the last query has no output: it skips, and reads no mask entry)
    if (pad != ~0ull &&
        (a.blocks == nullptr ||
         (q0 + 32 * wave < n && a.blocks[((long)h * a.n_qb + (q0 + 32 * wave) / 64) * a.n_kb + t]))) {
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
    const bool full = pad == 0 && mk.all_visible(q0 + off, q_last + off, j0, j0 + kKStep);
    unsigned dsk[2][8];
    unsigned rw[2][4][2];   // DROPOUT: this query's draws for each block's four runs of keys
    if constexpr (DROPOUT) {
      a.drop.runs4(bh, qi, j0 + 4 * hi, rw[0]);
      a.drop.runs4(bh, qi, j0 + 32 + 4 * hi, rw[1]);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float d2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float x = __builtin_fmaf(sc[mb][i + e], c, cm);
          if constexpr (ALIBI) {
            const int j = j0 + 32 * mb + 8 * ((i + e) >> 2) + 4 * hi + ((i + e) & 3);
            x = __builtin_fmaf(-b2, __builtin_fabsf((float)(qi + off - j)), x);
          }
          float p = exp2_fast(x);
          if (!full) {
            const int jt = 32 * mb + 8 * ((i + e) >> 2) + 4 * hi + ((i + e) & 3);
            p = (row_ok && mk.visible(qi + off, j0 + jt) && ((pad >> jt) & 1ull) == 0) ? p : 0.f;
          }
          if constexpr (DROPOUT) {   // key j: half e of word rw[i >> 2][(i & 3) >> 1]
            const bool kept = a.drop.keep_half(rw[mb][i >> 2][(i & 3) >> 1], e);
            d2[e] = p * ((kept ? dp[mb][i + e] * a.drop.scale : 0.f) + ndlt);
          } else {
            d2[e] = p * (dp[mb][i + e] + ndlt);
          }
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
    }   // selected block

    if (t_next < t_end) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    t = t_next;
  }

  if (row_ok) {
    char* row = a.dq + b * a.dq_bs + h * a.dq_hs + (long)qi * a.dq_rs;
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
  a.cu = p.cu;
  a.total = p.total;
  a.slopes = nullptr;
  a.drop = Dropout{0u, 0u, 0u, 0u, 1.f};
  a.blocks = nullptr;
  a.kpm = nullptr;
  a.n_qb = a.n_kb = 0;
  // dense [B, H, N, D], or a packed batch's [H, total, D] (sequence b starts at row cu[b])
  const long long row = (long long)p.D * 2;
  const long long head = (long long)(p.cu != nullptr ? p.total : p.N) * row;
  const long long batch = p.cu != nullptr ? 0 : p.H * head;
  a.q_bs = a.k_bs = a.v_bs = a.o_bs = a.g_bs = a.dq_bs = a.dk_bs = a.dv_bs = batch;
  a.q_hs = a.k_hs = a.v_hs = a.o_hs = a.g_hs = a.dq_hs = a.dk_hs = a.dv_hs = head;
  a.q_rs = a.k_rs = a.v_rs = a.o_rs = a.g_rs = a.dq_rs = a.dk_rs = a.dv_rs = (int)row;
  a.heads = p.H;
  a.n = p.N;
  a.nk = p.N;
  a.off = 0;
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
  // padded and packed batches always take the main kernels
  const bool main_kernels = env_bwd_choice() != 2 || p.seqlens != nullptr || p.cu != nullptr;
  // statistics and dQ in one call: the main dQ kernel forms the statistics of its own queries
  // (the same values, bit for bit, as the statistics pass) and runs first
  const bool fused = (stages & kBwdDelta) && (stages & kBwdDq) && main_kernels;
  if (fused) {
    if (hipError_t e = launch_dq_main(p, stream, /*form_stats=*/true); e != hipSuccess) return e;
  } else if (stages & kBwdDelta) {
    const unsigned gx = (unsigned)((stat_blocks(a.n) * kStatRows + 255) / 256);
    const unsigned gy = (unsigned)std::min(a.n_bh, 65535);
    if (p.seqlens != nullptr || p.cu != nullptr)
      hipLaunchKernelGGL((delta_kernel<D, BF16, true>), dim3(gx, gy), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((delta_kernel<D, BF16, false>), dim3(gx, gy), dim3(256), 0, stream, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  if ((stages & kBwdDkDv) && main_kernels) {
    if (hipError_t e = launch_dkdv_main(p, stream); e != hipSuccess) return e;
  } else if (stages & kBwdDkDv) {
    a.n_tiles = (a.n + kKvRows - 1) / kKvRows;
    hipLaunchKernelGGL((dkdv_kernel<D, BF16, false, false>), dim3((unsigned)((long)a.n_bh * a.n_tiles)),
                       dim3(256), 0, stream, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  if ((stages & kBwdDq) && main_kernels && !fused) {
    if (hipError_t e = launch_dq_main(p, stream); e != hipSuccess) return e;
  } else if ((stages & kBwdDq) && !fused) {
    a.n_tiles = (a.n + kDqRows - 1) / kDqRows;
    hipLaunchKernelGGL((dq_kernel<D, BF16, false, false>), dim3((unsigned)((long)a.n_bh * a.n_tiles)),
                       dim3(256), 0, stream, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D, bool BF16>
hipError_t launch_kv(const BwdKvParams& p, hipStream_t stream) {
  const long long e = 2;
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
  a.seqlens = nullptr;
  a.cu = nullptr;
  a.total = 0;
  a.slopes = p.slopes;
  a.drop = p.drop;
  a.blocks = p.blocks;
  a.kpm = p.kpm;
  a.n_qb = (p.Nq + 63) / 64;
  a.n_kb = (p.Nk + 63) / 64;
  const bool alibi = p.slopes != nullptr, drop = p.drop.scale != 1.f;
  a.q_bs = p.sq.b * e, a.q_hs = p.sq.h * e, a.q_rs = (int)(p.sq.r * e);
  a.k_bs = p.sk.b * e, a.k_hs = p.sk.h * e, a.k_rs = (int)(p.sk.r * e);
  a.v_bs = p.sv.b * e, a.v_hs = p.sv.h * e, a.v_rs = (int)(p.sv.r * e);
  a.o_bs = p.so.b * e, a.o_hs = p.so.h * e, a.o_rs = (int)(p.so.r * e);
  a.g_bs = p.sg.b * e, a.g_hs = p.sg.h * e, a.g_rs = (int)(p.sg.r * e);
  a.dq_bs = p.sdq.b * e, a.dq_hs = p.sdq.h * e, a.dq_rs = (int)(p.sdq.r * e);
  a.dk_bs = p.sdk.b * e, a.dk_hs = p.sdk.h * e, a.dk_rs = (int)(p.sdk.r * e);
  a.dv_bs = p.sdv.b * e, a.dv_hs = p.sdv.h * e, a.dv_rs = (int)(p.sdv.r * e);
  a.heads = p.H;
  a.n = p.Nq;
  a.nk = p.Nk;
  a.off = p.Nk - p.Nq;
  a.n_bh = p.B * p.H;
  a.sigma = softmax_sigma(p.scale);
  a.c = (float)((double)a.sigma * 1.4426950408889634);
  a.scale = p.scale;
  a.causal = p.causal;
  a.wl = p.window_left;
  a.wr = p.causal ? 0 : p.window_right;
  // dense operands, nothing extra but one of ALiBi, a block mask and a key padding mask, and
  // query tiles enough to fill the chip: the dK/dV and dQ kernels of fa_bwd (their band of visible query - key
  // differences shifted by N_k - N_q) (ALiBi only where no visible pair lies past the diagonal:
  // those kernels take its penalty as linear in the query - key distance)
  const bool alibi_main = !alibi || p.causal || p.window_right == 0;
  const int extras = alibi + (p.blocks != nullptr) + (p.kpm != nullptr);
  const bool lists_main = (p.blocks == nullptr && p.kpm == nullptr) || bwd_main_takes_blocks(p.Nq, p.Nk);
  const bool main = alibi_main && extras <= 1 && lists_main && !drop && p.Nq > 0 && p.Nk > 0 &&
                    (long)p.B * p.H * ((p.Nq + 127) / 128) >= 256 && is_dense(p.sq, p.H, p.Nq, p.D) &&
                    is_dense(p.so, p.H, p.Nq, p.D) && is_dense(p.sg, p.H, p.Nq, p.D) &&
                    is_dense(p.sdq, p.H, p.Nq, p.D) && is_dense(p.sk, p.H, p.Nk, p.D) &&
                    is_dense(p.sv, p.H, p.Nk, p.D) && is_dense(p.sdk, p.H, p.Nk, p.D) &&
                    is_dense(p.sdv, p.H, p.Nk, p.D);
  // the row statistics: formed by the main dQ kernel (which then runs first), else by their own
  // pass.  With no query, only dK = dV = 0 is left to write (the dK/dV kernel sees no query
  // step); with no key, dQ = 0
  if (!main && p.Nq > 0) {
    const unsigned gx = (unsigned)((stat_blocks(a.n) * kStatRows + 255) / 256);
    const unsigned gy = (unsigned)std::min(a.n_bh, 65535);
    hipLaunchKernelGGL((delta_kernel<D, BF16, false>), dim3(gx, gy), dim3(256), 0, stream, a);
    if (hipError_t err = hipGetLastError(); err != hipSuccess) return err;
  }
  if (main) {
    BwdParams m;
    m.q = p.q;
    m.k = p.k;
    m.v = p.v;
    m.o = p.o;
    m.dout = p.dout;
    m.lse = p.lse;
    m.dq = p.dq;
    m.dk = p.dk;
    m.dv = p.dv;
    m.stats = p.stats;
    m.seqlens = nullptr;
    m.cu = nullptr;
    m.slopes = p.slopes;
    m.blocks = p.blocks;
    m.kpm = p.kpm;
    m.B = p.B;
    m.H = p.H;
    m.N = p.Nq;
    m.D = p.D;
    m.bf16 = p.bf16;
    m.scale = p.scale;
    m.causal = p.causal;
    m.window_left = p.window_left;
    m.window_right = p.window_right;
    if (hipError_t err = launch_dq_main_kv(m, p.Nq, p.Nk, stream, /*form_stats=*/true); err != hipSuccess)
      return err;
    return launch_dkdv_main_kv(m, p.Nq, p.Nk, stream);
  }
  if (p.Nk > 0) {
    a.n_tiles = (p.Nk + kKvRows - 1) / kKvRows;
    const dim3 grid((unsigned)((long)a.n_bh * a.n_tiles));
    if (alibi && drop)
      hipLaunchKernelGGL((dkdv_kernel<D, BF16, true, true>), grid, dim3(256), 0, stream, a);
    else if (alibi)
      hipLaunchKernelGGL((dkdv_kernel<D, BF16, true, false>), grid, dim3(256), 0, stream, a);
    else if (drop)
      hipLaunchKernelGGL((dkdv_kernel<D, BF16, false, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((dkdv_kernel<D, BF16, false, false>), grid, dim3(256), 0, stream, a);
    if (hipError_t err = hipGetLastError(); err != hipSuccess) return err;
  }
  if (p.Nq == 0) return hipSuccess;
  a.n_tiles = (p.Nq + kDqRows - 1) / kDqRows;
  const dim3 grid((unsigned)((long)a.n_bh * a.n_tiles));
  if (alibi && drop)
    hipLaunchKernelGGL((dq_kernel<D, BF16, true, true>), grid, dim3(256), 0, stream, a);
  else if (alibi)
    hipLaunchKernelGGL((dq_kernel<D, BF16, true, false>), grid, dim3(256), 0, stream, a);
  else if (drop)
    hipLaunchKernelGGL((dq_kernel<D, BF16, false, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((dq_kernel<D, BF16, false, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_kv(const BwdKvParams& p, hipStream_t stream) {
  if (p.D == 64) return p.bf16 ? launch_kv<64, true>(p, stream) : launch_kv<64, false>(p, stream);
  return p.bf16 ? launch_kv<128, true>(p, stream) : launch_kv<128, false>(p, stream);
}

hipError_t launch_bwd(const BwdParams& p, unsigned stages, hipStream_t stream) {
  if (p.D == 64) return p.bf16 ? launch<64, true>(p, stages, stream) : launch<64, false>(p, stages, stream);
  return p.bf16 ? launch<128, true>(p, stages, stream) : launch<128, false>(p, stages, stream);
}

}  // namespace fa
