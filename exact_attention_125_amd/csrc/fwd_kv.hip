// N_q queries over N_k keys for gfx950: the plan, the few-query (decode) kernel, and the merge
// of key splits.
//
// Query i sits at key position i + (N_k - N_q), so the queries are the last N_q positions of
// the key sequence: a decode step of an LLM over its KV cache (the inference use of "Flash
// Attention 3.7 核心原理与实战" §1.3; the KV cache PagedAttention pages through memory, closing
// section of "PyTorch-CUDA-v2.9镜像中使用FlashAttention提升训练速度") sees every cached key, and
// a block of new queries sees the cache plus its own causal prefix.  Operands may have any
// strides with a contiguous head dimension, e.g. the (batch, seq, heads, head_dim) memory
// behind the transposed views of that page's §4.2 module.
//
// Few queries (N_q <= kDecodeMaxQ): every key row is read once and used for at most four dot
// products, so the work is bound by HBM bandwidth, not by a matrix product; the kernel uses
// no MFMA.  A workgroup takes one (batch, head) and one split of its keys.  Each key row is
// D/8 lanes of 16 bytes, so a load instruction of a wave reads whole consecutive rows; the
// lanes of a row add their partial dot products with DPP butterflies (every lane ends with
// the same sum).  The row groups of a workgroup each run their own running max / running sum
// over their rows ("告别OOM和训练慢" §2.2, in base 2), four rows per step with the loads of the
// next step in flight, and merge through LDS at the end.  With several splits each writes a
// normalised partial O and its LSE, and combine_kernel merges them by the log-sum-exp rule
//     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
// which is exact because each O_s is a softmax-weighted mean over disjoint key sets.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "cdna4.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecU = 4;   // key rows per row group and step (16-bit keys)

// Key rows per step: D / 8 lanes per row; an FP8 cache (8-byte lane loads) takes twice the rows
// per step, so a step keeps as many bytes in flight.
__host__ __device__ constexpr int dec_step_rows(int d, bool fp8 = false) {
  return kDecThreads / (d / 8) * kDecU * (fp8 ? 2 : 1);
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct DecArgs {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  long long q_bs, q_hs, k_bs, k_hs, v_bs, v_hs, o_bs, o_hs;   // bytes
  int q_rs, k_rs, v_rs, o_rs;                                 // bytes
  int nq, nk, off, n_h, n_bh, n_split, split_keys;
  float* po;      // n_split > 1: partial O [n_split, B*H, nq, D] and LSE [n_split, B*H, nq]
  float* plse;
  const float* slopes;   // ALiBi slopes [heads] (device), or null
  const unsigned char* brow0;   // block-sparse mask [heads][n_qb][n_kb] (queries < 64: row 0)
  const unsigned char* kpm;     // key padding mask [B][nk] (nonzero = padding key), or null
  int n_qb, n_kb;
  float c;        // softmax_scale * log2(e) (* the key descale of an FP8 cache), signed
  float vs;       // the value descale of an FP8 cache (1 otherwise)
  int causal, wl, wr;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dec_rsrc(const char* base, int rows, int rs,
                                                           int row_bytes) {
  return make_rsrc(base, rows > 0 ? (rows - 1) * rs + row_bytes : 0);
}

template <bool BF16>
__device__ __forceinline__ void unpack8(u32x4 x, float (&f)[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const unsigned word = x[w];
    f[2 * w] = to_float<BF16>((unsigned short)(word & 0xffffu));
    f[2 * w + 1] = to_float<BF16>((unsigned short)(word >> 16));
  }
}

// Eight FP8 E4M3 codes (the OCP 8-bit format: 4 exponent bits, bias 7, 3 mantissa bits) of
// one key or value row, lowest address first, widened exactly to float by the hardware.
__device__ __forceinline__ void unpack8_fp8(u32x2 x, float (&f)[8]) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[w], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[w], true);
    f[4 * w] = lo[0];
    f[4 * w + 1] = lo[1];
    f[4 * w + 2] = hi[0];
    f[4 * w + 3] = hi[1];
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_read(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the G consecutive lanes of a row group (G = 8 or 16, aligned), left in every one of
// them.  Each stage adds a value to its mirror image, so all lanes compute the same sums in the
// same order and end bit-identical.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_read<0xB1>(x);     // quad_perm [1, 0, 3, 2]
  x += dpp_read<0x4E>(x);     // quad_perm [2, 3, 0, 1]
  x += dpp_read<0x141>(x);    // row_half_mirror: quads 0 <-> 1 of each 8 lanes
  if constexpr (G == 16) x += dpp_read<0x140>(x);   // row_mirror: halves of 16 lanes
  return x;
}

// FP8: keys and values are FP8 E4M3 codes (one byte per element, 8 bytes per lane); the key
// descale is folded into a.c and the value descale a.vs scales the normalised output.
template <int D, bool BF16, int NQ, bool FP8>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecArgs a) {
  constexpr int G = D / 8;                      // lanes per key row, 8 elements each
  constexpr int GROUPS = kDecThreads / G;       // rows per load instruction of the workgroup
  // rows per group and step: an FP8 cache takes twice as many (the same bytes), except at
  // N_q > 2, where the scores of a step would not fit the registers
  constexpr int U = FP8 && NQ <= 2 ? 2 * kDecU : kDecU;
  constexpr int STEP = GROUPS * U;              // rows per step
  constexpr int kElt = FP8 ? 1 : 2;             // bytes per key / value element
  constexpr int kRowBytes = D * kElt;
  using KV = std::conditional_t<FP8, u32x2, u32x4>;   // one lane's 8 elements of a row
  static_assert(STEP * (FP8 && NQ > 2 ? 2 : 1) == dec_step_rows(D, FP8), "step size");

  __shared__ float sm_m[GROUPS][NQ];
  __shared__ float sm_l[GROUPS][NQ];
  __shared__ __attribute__((aligned(16))) float sm_o[GROUPS][NQ][D];

  const int tid = threadIdx.x;
  const int grp = tid / G, cl = tid % G;
  const int bh = blockIdx.x / a.n_split, split = blockIdx.x - bh * a.n_split;
  const int b = bh / a.n_h, h = bh - b * a.n_h;
  const int nq = a.nq, nk = a.nk, off = a.off;
  const float NEG_INF = -__builtin_inff();
  const float b2 = a.slopes != nullptr ? a.slopes[h] * kLog2e : 0.f;   // ALiBi, base 2

  // keys of this split that some query can see
  const Mask mk{nk, a.causal, a.wl, a.wr};
  int lo, hi;
  mk.key_range(off, nq - 1 + off, lo, hi);
  lo = max(lo, split * a.split_keys);
  hi = min(hi, (split + 1) * a.split_keys);
  const bool all_vis = lo < hi && mk.all_visible(off, nq - 1 + off, lo, hi) && a.brow0 == nullptr &&
                       a.kpm == nullptr;
  // block-sparse: the (single, nq <= 4 < 64) query block's row of the mask
  const unsigned char* brow = a.brow0 ? a.brow0 + (long)h * a.n_qb * a.n_kb : nullptr;
  // key padding: this batch entry's row of the mask
  const unsigned char* kpm = a.kpm ? a.kpm + (long)b * nk : nullptr;
  const int n_steps = lo < hi ? (hi - lo + STEP - 1) / STEP : 0;

  // the queries' 8 elements of this lane, times c (so scores come out in base-2 units)
  float qf[NQ][8];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    if (qi < nq) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(a.q + b * a.q_bs + h * a.q_hs +
                                                      (long)qi * a.q_rs + cl * 16);
      unpack8<BF16>(x, qf[qi]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[qi][e] *= a.c;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[qi][e] = 0.f;
    }
  }

  const auto rk = dec_rsrc(a.k + b * a.k_bs + h * a.k_hs, nk, a.k_rs, kRowBytes);
  const auto rv = dec_rsrc(a.v + b * a.v_bs + h * a.v_hs, nk, a.v_rs, kRowBytes);

  float m[NQ], l[NQ], o[NQ][8];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    m[qi] = NEG_INF;
    l[qi] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[qi][e] = 0.f;
  }

  auto load = [&](KV (&kb)[U], KV (&vb)[U], int r0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * GROUPS + grp;
      if constexpr (FP8) {
        kb[u] = __builtin_amdgcn_raw_buffer_load_b64(rk, r * a.k_rs + cl * 8, 0, 0);
        vb[u] = __builtin_amdgcn_raw_buffer_load_b64(rv, r * a.v_rs + cl * 8, 0, 0);
      } else {
        kb[u] = buffer_load16(rk, r * a.k_rs + cl * 16);
        vb[u] = buffer_load16(rv, r * a.v_rs + cl * 16);
      }
    }
  };
  auto unpack_kv = [](const KV& x, float (&f)[8]) {
    if constexpr (FP8)
      unpack8_fp8(x, f);
    else
      unpack8<BF16>(x, f);
  };

  // One step: U rows of this group.  MASKED hides rows past hi and rows a query cannot see.
  auto step = [&](auto masked_tag, const KV (&kb)[U], const KV (&vb)[U], int r0) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float s[NQ][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
      unpack_kv(kb[u], kf);
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
        float part = qf[qi][0] * kf[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) part = __builtin_fmaf(qf[qi][e], kf[e], part);
        s[qi][u] = group_sum<G>(part);
      }
      // ALiBi penalty -slope |p - j| (zero without slopes)
      const int r = r0 + u * GROUPS + grp;
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi)
        s[qi][u] = __builtin_fmaf(-b2, __builtin_fabsf((float)(qi + off - r)), s[qi][u]);
      if constexpr (MASKED) {
        const bool in_block = (brow == nullptr || (r < hi && brow[r >> 6])) &&
                              (kpm == nullptr || (r < hi && kpm[r] == 0));
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi)
          s[qi][u] = (r < hi && in_block && mk.visible(qi + off, r)) ? s[qi][u] : NEG_INF;
      }
    }
    float p[NQ][U];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      float mx = m[qi];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[qi][u]);
      const float mu = mx == NEG_INF ? 0.f : mx;
      const float alpha = exp2_fast(m[qi] - mu);   // 0 while nothing was seen
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[qi][u] = exp2_fast(s[qi][u] - mu);
        sum += p[qi][u];
      }
      l[qi] = __builtin_fmaf(l[qi], alpha, sum);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[qi][e] *= alpha;
      m[qi] = mx;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
      unpack_kv(vb[u], vf);
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[qi][e] = __builtin_fmaf(p[qi][u], vf[e], o[qi][e]);
    }
  };

  auto run = [&](const KV (&kb)[U], const KV (&vb)[U], int r0) {
    if (all_vis && r0 + STEP <= hi)
      step(std::false_type{}, kb, vb, r0);
    else
      step(std::true_type{}, kb, vb, r0);
  };

  // Register sets in a ring: the loads of the next one (N_q = 4: register room for one) or two
  // steps are in flight while a step is computed.
  KV ka[U], va[U], kb2[U], vb2[U];
  if constexpr (NQ <= 2) {
    KV kc[U], vc[U];
    if (n_steps > 0) load(ka, va, lo);
    if (n_steps > 1) load(kb2, vb2, lo + STEP);
    for (int t = 0; t < n_steps; t += 3) {
      if (t + 2 < n_steps) load(kc, vc, lo + (t + 2) * STEP);
      run(ka, va, lo + t * STEP);
      if (t + 3 < n_steps) load(ka, va, lo + (t + 3) * STEP);
      if (t + 1 < n_steps) run(kb2, vb2, lo + (t + 1) * STEP);
      if (t + 4 < n_steps) load(kb2, vb2, lo + (t + 4) * STEP);
      if (t + 2 < n_steps) run(kc, vc, lo + (t + 2) * STEP);
    }
  } else {
    if (n_steps > 0) load(ka, va, lo);
    for (int t = 0; t < n_steps; t += 2) {
      if (t + 1 < n_steps) load(kb2, vb2, lo + (t + 1) * STEP);
      run(ka, va, lo + t * STEP);
      if (t + 2 < n_steps) load(ka, va, lo + (t + 2) * STEP);
      if (t + 1 < n_steps) run(kb2, vb2, lo + (t + 1) * STEP);
    }
  }

  // ---- merge the row groups
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    *reinterpret_cast<f32x4*>(&sm_o[grp][qi][cl * 8]) = f32x4{o[qi][0], o[qi][1], o[qi][2], o[qi][3]};
    *reinterpret_cast<f32x4*>(&sm_o[grp][qi][cl * 8 + 4]) =
        f32x4{o[qi][4], o[qi][5], o[qi][6], o[qi][7]};
    if (cl == 0) {
      sm_m[grp][qi] = m[qi];
      sm_l[grp][qi] = l[qi];
    }
  }
  __syncthreads();
  for (int t = tid; t < NQ * D; t += kDecThreads) {
    const int qi = t / D, e = t - qi * D;
    if (qi >= nq) break;
    float mx = NEG_INF;
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) mx = fmaxf(mx, sm_m[g][qi]);
    const float mu = mx == NEG_INF ? 0.f : mx;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) {
      const float w = exp2_fast(sm_m[g][qi] - mu);
      L = __builtin_fmaf(w, sm_l[g][qi], L);
      O = __builtin_fmaf(w, sm_o[g][qi][e], O);
    }
    const bool live = L > 0.f;
    const float val = live ? (FP8 ? O / L * a.vs : O / L) : 0.f;
    const float lse = live ? (mx + __builtin_log2f(L)) * kLn2 : NEG_INF;
    if (a.n_split == 1) {
      char* orow = a.o + b * a.o_bs + h * a.o_hs + (long)qi * a.o_rs;
      *reinterpret_cast<unsigned short*>(orow + 2 * e) = (unsigned short)(pack2<BF16>(val, 0.f) & 0xffffu);
      if (e == 0 && a.lse != nullptr) a.lse[(long)bh * nq + qi] = lse;
    } else {
      const long prow = ((long)split * a.n_bh + bh) * nq + qi;
      a.po[prow * D + e] = val;
      if (e == 0) a.plse[prow] = lse;
    }
  }
}

struct CombineArgs {
  const float* po;
  const float* plse;
  char* o;
  float* lse;
  long long o_bs, o_hs;
  int o_rs;
  int nq, n_h, n_bh, n_split;
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// One wave per (batch, head, query): merges the splits' partial results, 16 splits at a time.
// The LSEs of a group (one per lane) and its partial rows are loaded together, so a group
// costs one memory round trip; the groups are merged with a running maximum.
template <int D, bool BF16>
__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a) {
  constexpr int E = D / 64;   // elements per lane
  constexpr int kGroup = 16;
  const int lane = threadIdx.x;
  const int row = blockIdx.x;                 // bh * nq + qi
  const int bh = row / a.nq, qi = row - bh * a.nq;
  const int b = bh / a.n_h, h = bh - b * a.n_h;
  const long stride = (long)a.n_bh * a.nq;    // between splits, in rows
  const float NEG_INF = -__builtin_inff();
  float mx = NEG_INF, L = 0.f, O[E];
#pragma unroll
  for (int i = 0; i < E; ++i) O[i] = 0.f;
  for (int s0 = 0; s0 < a.n_split; s0 += kGroup) {
    const int n = min(kGroup, a.n_split - s0);
    const float ls = lane < n ? a.plse[(s0 + lane) * stride + row] : NEG_INF;
    const float* po = a.po + ((long)s0 * stride + row) * D + lane;
    float pv[kGroup][E];
#pragma unroll
    for (int j = 0; j < kGroup; ++j)
#pragma unroll
      for (int i = 0; i < E; ++i) pv[j][i] = j < n ? po[j * stride * D + 64 * i] : 0.f;
    const float m_new = fmaxf(mx, wave_max(ls));
    const float mu = m_new == NEG_INF ? 0.f : m_new;
    const float alpha = exp2_fast((mx - mu) * kLog2e);   // 0 before the first live split
    const float w = exp2_fast((ls - mu) * kLog2e);        // 0 for lanes without a split
    L = __builtin_fmaf(L, alpha, w);                       // per lane; summed at the end
#pragma unroll
    for (int i = 0; i < E; ++i) O[i] *= alpha;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const float wj = __shfl(w, j);
#pragma unroll
      for (int i = 0; i < E; ++i) O[i] = __builtin_fmaf(wj, pv[j][i], O[i]);
    }
    mx = m_new;
  }
  L = wave_sum(L);
  const bool live = L > 0.f;
  const float inv = live ? 1.f / L : 0.f;
  char* orow = a.o + b * a.o_bs + h * a.o_hs + (long)qi * a.o_rs;
#pragma unroll
  for (int i = 0; i < E; ++i)
    *reinterpret_cast<unsigned short*>(orow + 2 * (lane + 64 * i)) =
        (unsigned short)(pack2<BF16>(O[i] * inv, 0.f) & 0xffffu);
  if (lane == 0 && a.lse != nullptr) a.lse[row] = live ? mx + __builtin_logf(L) : NEG_INF;
}

template <int D, bool BF16, bool FP8>
hipError_t launch_decode(const KvParams& p, const KvPlan& plan, hipStream_t stream) {
  const long long e = 2, ekv = FP8 ? 1 : 2;   // bytes per element: queries / outputs, keys / values
  DecArgs a;
  a.q = static_cast<const char*>(p.q);
  a.k = static_cast<const char*>(p.k);
  a.v = static_cast<const char*>(p.v);
  a.o = static_cast<char*>(p.o);
  a.lse = p.lse;
  a.q_bs = p.sq.b * e, a.q_hs = p.sq.h * e, a.q_rs = (int)(p.sq.r * e);
  a.k_bs = p.sk.b * ekv, a.k_hs = p.sk.h * ekv, a.k_rs = (int)(p.sk.r * ekv);
  a.v_bs = p.sv.b * ekv, a.v_hs = p.sv.h * ekv, a.v_rs = (int)(p.sv.r * ekv);
  a.o_bs = p.so.b * e, a.o_hs = p.so.h * e, a.o_rs = (int)(p.so.r * e);
  a.nq = p.Nq;
  a.nk = p.Nk;
  a.off = p.Nk - p.Nq;
  a.n_h = p.H;
  a.n_bh = p.B * p.H;
  a.n_split = plan.n_split;
  a.split_keys = plan.split_keys;
  a.po = p.ws;
  a.plse = p.ws ? p.ws + (size_t)plan.n_split * a.n_bh * p.Nq * D : nullptr;
  a.slopes = p.slopes;
  a.brow0 = p.blocks;
  a.kpm = p.kpm;
  a.n_qb = (p.Nq + 63) / 64;
  a.n_kb = (p.Nk + 63) / 64;
  a.c = (float)((double)p.scale * 1.4426950408889634 * (FP8 ? (double)p.k_descale : 1.0));
  a.vs = FP8 ? p.v_descale : 1.f;
  a.causal = p.causal;
  a.wl = p.window_left;
  a.wr = p.causal ? 0 : p.window_right;
  const dim3 grid((unsigned)((long)a.n_bh * a.n_split));
  if (p.Nq == 1)
    hipLaunchKernelGGL((decode_kernel<D, BF16, 1, FP8>), grid, dim3(kDecThreads), 0, stream, a);
  else if (p.Nq == 2)
    hipLaunchKernelGGL((decode_kernel<D, BF16, 2, FP8>), grid, dim3(kDecThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, BF16, kDecodeMaxQ, FP8>), grid, dim3(kDecThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_combine(const KvParams& p, const KvPlan& plan, hipStream_t stream) {
  CombineArgs a;
  a.po = p.ws;
  a.plse = p.ws + (size_t)plan.n_split * p.B * p.H * p.Nq * D;
  a.o = static_cast<char*>(p.o);
  a.lse = p.lse;
  a.o_bs = p.so.b * 2, a.o_hs = p.so.h * 2, a.o_rs = (int)(p.so.r * 2);
  a.nq = p.Nq;
  a.n_h = p.H;
  a.n_bh = p.B * p.H;
  a.n_split = plan.n_split;
  hipLaunchKernelGGL((combine_kernel<D, BF16>), dim3((unsigned)((long)a.n_bh * p.Nq)), dim3(64), 0,
                     stream, a);
  return hipGetLastError();
}

long ceil_div(long a, long b) { return (a + b - 1) / b; }

}  // namespace

KvPlan kv_plan(int B, int H, int Nq, int Nk, int D, bool dropout, bool fp8) {
  KvPlan p{};
  const long bh = (long)B * H;
  long split_keys;
  if (Nq <= kDecodeMaxQ && !dropout) {
    // about 512 workgroups: one round at two per CU, so each workgroup's start (query load,
    // first key rows) and end (merge, stores) latency is paid once per CU pair; at least four
    // steps of keys each
    p.decode = true;
    const long step = dec_step_rows(D, fp8);
    const long want = ceil_div(512, bh > 0 ? bh : 1);
    split_keys = ceil_div(ceil_div(Nk, want), step) * step;
    if (split_keys < 4 * step) split_keys = 4 * step;
  } else {
    // split the keys only when the query tiles leave most of the chip idle
    p.decode = false;
    const long wgs = bh * ceil_div(Nq, 128);
    long n = 1;
    if (wgs < 512 && Nk > 1024) n = std::min(ceil_div(512, wgs), ceil_div(Nk, 512));
    split_keys = ceil_div(ceil_div(Nk > 0 ? Nk : 1, n), kKvMfmaKeyStep) * kKvMfmaKeyStep;
  }
  p.split_keys = (int)split_keys;
  p.n_split = Nk > 0 ? (int)ceil_div(Nk, split_keys) : 1;
  p.ws_bytes = p.n_split > 1 ? (size_t)p.n_split * bh * Nq * (D + 1) * sizeof(float) : 0;
  return p;
}

hipError_t launch_fwd_kv(const KvParams& p, const KvPlan& plan, hipStream_t stream) {
  // dense operands, nothing extra but one of ALiBi, a block mask and a key padding mask, one key
  // split, and query tiles enough to fill the chip: the main forward kernel
  const int extras = (p.slopes != nullptr) + (p.blocks != nullptr) + (p.kpm != nullptr);
  if (!plan.decode && !p.fp8 && plan.n_split == 1 && extras <= 1 &&
      ((p.blocks == nullptr && p.kpm == nullptr) || fwd_main_takes_blocks(p.D, p.Nk)) &&
      p.drop.scale == 1.f && p.Nk > 0 && (long)p.B * p.H * ((p.Nq + 127) / 128) >= 256 &&
      is_dense(p.sq, p.H, p.Nq, p.D) && is_dense(p.so, p.H, p.Nq, p.D) &&
      is_dense(p.sk, p.H, p.Nk, p.D) && is_dense(p.sv, p.H, p.Nk, p.D))
    return launch_fwd_main_kv(p, stream);
  hipError_t e;
  if (plan.decode && p.fp8) {
    if (p.D == 64)
      e = p.bf16 ? launch_decode<64, true, true>(p, plan, stream)
                 : launch_decode<64, false, true>(p, plan, stream);
    else
      e = p.bf16 ? launch_decode<128, true, true>(p, plan, stream)
                 : launch_decode<128, false, true>(p, plan, stream);
  } else if (p.fp8) {
    return hipErrorInvalidValue;   // an FP8 cache is read by the few-query kernel only
  } else if (plan.decode) {
    if (p.D == 64)
      e = p.bf16 ? launch_decode<64, true, false>(p, plan, stream)
                 : launch_decode<64, false, false>(p, plan, stream);
    else
      e = p.bf16 ? launch_decode<128, true, false>(p, plan, stream)
                 : launch_decode<128, false, false>(p, plan, stream);
  } else {
    e = launch_fwd_kv_mfma(p, plan, stream);
  }
  if (e != hipSuccess || plan.n_split == 1) return e;
  if (p.D == 64)
    return p.bf16 ? launch_combine<64, true>(p, plan, stream) : launch_combine<64, false>(p, plan, stream);
  return p.bf16 ? launch_combine<128, true>(p, plan, stream) : launch_combine<128, false>(p, plan, stream);
}

}  // namespace fa
