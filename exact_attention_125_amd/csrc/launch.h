// Internal interface between the validating C-ABI layer (api.cpp) and the kernel
// launchers (fwd.hip, bwd.hip).  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "cdna4.h"

namespace fa {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // may be null
  const int* seqlens = nullptr;   // device int32[B], or null: sequence b is rows
                                  // 0 .. seqlens[b]-1 of its N (values clamped to [0, N]);
                                  // the rest is padding
  const int* cu = nullptr;        // device int32[B + 1], or null: a packed batch, sequence b is
                                  // rows cu[b] .. cu[b+1]-1 of each head's `total` rows
                                  // ([H, total, D] arrays; N is the longest sequence)
  int total = 0;
  int B, H, N, D;
  bool bf16;
  float scale;         // softmax scale
  int causal;
  int window_left;     // -1 = unbounded
  int window_right;    // -1 = unbounded (ignored when causal)
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* stats;        // workspace: per-query statistics in 32-query blocks (stat_index)
  const int* seqlens = nullptr;   // as in FwdParams
  const int* cu = nullptr;        // as in FwdParams
  const float* slopes = nullptr;  // ALiBi slopes [H] (device), or null: the main dK/dV and dQ
                                  // kernels take them where no visible pair lies past the
                                  // diagonal (causal, or a right window of 0)
  const unsigned char* blocks = nullptr;   // block-sparse mask [H][ceil(N_q/64)][ceil(N_k/64)]
                                           // (device), or null; not with slopes
  const unsigned char* kpm = nullptr;      // key padding mask [B][N_k] (device), or null; not
                                           // with slopes or blocks
  int total = 0;
  int B, H, N, D;
  bool bf16;
  float scale;
  int causal;
  int window_left;
  int window_right;
};

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);

// Forward over FP8 E4M3 Q, K, V codes (dense [B, H, N, D], one byte per element) with one
// descale factor per tensor; O is fp16 or bf16, LSE fp32 (fwd_fp8.hip).
struct Fp8FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // may be null
  int B, H, N, D;
  bool out_bf16;
  float scale;         // softmax scale
  float q_descale, k_descale, v_descale;
  int causal;
  int window_left;
  int window_right;
};
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream);

// Strides of one [B, H, rows, d] operand, in elements (the last dimension is contiguous).
struct Strides {
  long long b, h, r;
};

// Whether s is the dense layout of [B, H, rows, D] (rows of D elements, heads of rows rows).
inline bool is_dense(const Strides& s, int H, int rows, int D) {
  return s.r == D && s.h == (long long)rows * D && s.b == (long long)H * rows * D;
}

// N_q queries over N_k keys: query i sits at key position i + (N_k - N_q).
struct KvParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // [B, H, N_q] dense, may be null
  float* ws;           // partial results of key splits (KvPlan::ws_bytes), null if none
  const float* slopes = nullptr;   // ALiBi slopes [H] (device), or null
  Dropout drop{0u, 0u, 0u, 0u, 1.f};   // scale 1: no dropout
  const unsigned char* blocks = nullptr;   // block-sparse mask [H][ceil(Nq/64)][ceil(Nk/64)]
  const unsigned char* kpm = nullptr;      // key padding mask [B][Nk], nonzero = padding key
  Strides sq, sk, sv, so;
  int B, H, Nq, Nk, D;
  bool bf16;
  bool fp8 = false;          // keys and values are FP8 E4M3 codes (the few-query kernel only)
  float k_descale = 1.f;     // FP8: key element = k_descale * code value
  float v_descale = 1.f;     // FP8: value element = v_descale * code value
  float scale;
  int causal;
  int window_left;
  int window_right;
};

// How a call is run: which kernel, how many key splits of how many keys, and the workspace
// their partial results take (0 with one split).  A function of the shape alone, so a
// call's rounding does not depend on the device.
struct KvPlan {
  bool decode;         // the few-query kernel (N_q <= kDecodeMaxQ) rather than the MFMA one
  int n_split;
  int split_keys;      // keys per split (a multiple of the kernel's key step)
  size_t ws_bytes;
};
constexpr int kDecodeMaxQ = 4;
constexpr int kKvMfmaKeyStep = 64;   // key tile of the four-wave MFMA kernel
// dropout: the few-query kernel has no dropout, so such calls take the MFMA kernel
// fp8: keys and values are FP8 codes (the few-query kernel then takes twice the rows per step).
KvPlan kv_plan(int B, int H, int Nq, int Nk, int D, bool dropout, bool fp8 = false);
// Runs the plan: the chosen kernel, then (with key splits) the merge of the partial results.
hipError_t launch_fwd_kv(const KvParams& p, const KvPlan& plan, hipStream_t stream);
// The main forward kernel (fwd_main.hip) for N_q queries over N_k keys, dense operands, with at
// most one of ALiBi slopes, a block mask and a key padding mask, and no dropout.
hipError_t launch_fwd_main_kv(const KvParams& p, hipStream_t stream);
// whether the main forward kernel takes a block-sparse or key padding mask over nk keys (its
// per-tile list holds them)
bool fwd_main_takes_blocks(int D, int nk);
// whether the main dK/dV and dQ kernels take a block-sparse or key padding mask over nq queries
// and nk keys (their step lists hold them)
inline bool bwd_main_takes_blocks(int nq, int nk) { return nq <= 32 * 1024 && nk <= 32 * 1024; }
// The MFMA kernel alone (fwd.hip); with plan.n_split > 1 it leaves partial results in p.ws.
hipError_t launch_fwd_kv_mfma(const KvParams& p, const KvPlan& plan, hipStream_t stream);
// The main forward (128 query rows per workgroup, direct global->LDS copies, two-phase
// software pipeline), for grids that fill the chip and for padded batches; launch_fwd chooses
// between it and the four-wave kernel of fwd.hip.
hipError_t launch_fwd_main(const FwdParams& p, hipStream_t stream);
// The forward for grids too small to fill the chip: 64 query rows per workgroup, the key loop
// split over 2 to 4 parts (one wave pair each) and merged in LDS (fwd_split.hip).
hipError_t launch_fwd_split(const FwdParams& p, hipStream_t stream);
// Backward stages, run in this order on one stream: the row statistics (log2(e) * LSE and
// delta = rowsum(dO * O)) into the workspace, then dK/dV, then dQ (both read them).
constexpr unsigned kBwdDelta = 1u, kBwdDkDv = 2u, kBwdDq = 4u, kBwdAll = 7u;
hipError_t launch_bwd(const BwdParams& p, unsigned stages, hipStream_t stream);

// Backward of fa_fwd_kv: N_q queries over N_k keys, any strides (the four-wave kernels).
struct BwdKvParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;    // [B, H, N_q] dense
  void* dq;
  void* dk;
  void* dv;
  float* stats;        // workspace, as for BwdParams with N = N_q
  const float* slopes = nullptr;   // ALiBi slopes [H] (device), or null
  Dropout drop{0u, 0u, 0u, 0u, 1.f};   // as in the forward call
  const unsigned char* blocks = nullptr;   // as in the forward call
  const unsigned char* kpm = nullptr;      // as in the forward call
  Strides sq, sk, sv, so, sg, sdq, sdk, sdv;
  int B, H, Nq, Nk, D;
  bool bf16;
  float scale;
  int causal;
  int window_left;
  int window_right;
};
hipError_t launch_bwd_kv(const BwdKvParams& p, hipStream_t stream);

// The backward passes evaluate P = exp(scale s - LSE) as 2^(c (s + m)) with c = sigma log2(e)
// and the per-row m = -LSE / sigma, where sigma is the scale moved away from zero (a zero
// scale leaves every score weight equal, which sigma = 1e-30 reproduces to fp32 rounding).
// Backward workspace layout: for each (batch, head) and each block of 32 queries, 64 floats:
// m = -LSE / sigma of the block's 32 queries, then their -rowsum(dO * O); zero for query
// slots past N.  A block's statistics are one contiguous 256-byte run, copied as one piece.
constexpr int kStatRows = 32;
__host__ __device__ inline int stat_blocks(int n) { return (n + kStatRows - 1) / kStatRows; }
// index of m of query q of head bh (add kStatRows for its -delta)
__host__ __device__ inline long stat_index(long bh, int n, int q) {
  return (bh * stat_blocks(n) + q / kStatRows) * (2 * kStatRows) + q % kStatRows;
}

inline float softmax_sigma(float scale) {
  constexpr float kTiny = 1e-30f;
  if (scale >= 0.f) return scale < kTiny ? kTiny : scale;
  return scale > -kTiny ? -kTiny : scale;
}
// dK/dV with key-owned workgroups of one wave per SIMD (bwd_dkdv.hip); launch_bwd chooses
// between it and the four-wave kernel of bwd.hip.
hipError_t launch_dkdv_main(const BwdParams& p, hipStream_t stream);
// dQ with query-owned workgroups of one wave per SIMD (bwd_dq.hip).  form_stats: the kernel
// forms the statistics of its queries itself (from p.o and p.lse) and writes them to p.stats,
// in place of the statistics pass; the dK/dV kernel then runs after it.
hipError_t launch_dq_main(const BwdParams& p, hipStream_t stream, bool form_stats = false);
// The same two kernels for nq query rows over nk key rows of dense [B, H, rows, D] operands
// (query i at key position i + nk - nq; p.N is ignored, no padded batch).
hipError_t launch_dkdv_main_kv(const BwdParams& p, int nq, int nk, hipStream_t stream);
hipError_t launch_dq_main_kv(const BwdParams& p, int nq, int nk, hipStream_t stream, bool form_stats = false);

}  // namespace fa
