// C ABI entry points (include/fa.h): argument validation, then kernel launch.
//
// Validation runs entirely on the host before any HIP call, so an invalid call enqueues
// nothing and every error path can be exercised without a GPU.
#include "../../include/fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

constexpr long kMaxRowElems = 1L << 30;   // N * d limit (32-bit byte offsets inside a head)
constexpr long kMaxRows = 1L << 31;       // B * H * N limit

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared checks of shape, head dim, dtype, window and scale.  Sets *empty when the call has
// no work (some dimension is zero).
fa_status check_common(int B, int H, int N, int d, fa_dtype dtype, float scale, int wl, int wr,
                       bool* empty) {
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_BAD_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_BAD_SHAPE;
  if ((long)N * d >= kMaxRowElems) return FA_ERR_BAD_SHAPE;
  if ((long)B * H * (long)N >= kMaxRows) return FA_ERR_BAD_SHAPE;
  if (wl < -1 || wr < -1) return FA_ERR_BAD_WINDOW;
  if (!std::isfinite(scale)) return FA_ERR_BAD_SCALE;
  *empty = (B == 0 || H == 0 || N == 0);
  return FA_OK;
}

fa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  g_last_error = hipGetErrorString(e);
  return FA_ERR_HIP;
}

// ---- static scratch of fa_bwd_noalloc
// One file-scope device array per GPU (each device the library runs on holds its own copy, at
// its own address, until the process ends).  In host code the array's name is only a host-side
// stand-in: the device address of a GPU's copy comes from hipGetSymbolAddress, asked once per
// device with that device current, and only that address is handed to the kernels.  Every
// call on a device shares its copy; the statistics pass overwrites every slot the later passes
// read (zeros past the sequence included), so nothing needs clearing, and calls that overlap
// on one device race on it.
constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];   // device address of each device's `scratch` (null: not asked yet)

// This device's copy (the calling thread's current device), or null after a HIP error.
void* scratch_of_current_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    hip_status(e);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_error = "device ordinal beyond the scratch table";
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      hip_status(e);
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int fa_version(void) { return 100; }

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL_PTR: return "FA_ERR_NULL_PTR: a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "FA_ERR_BAD_SHAPE: batch, heads or seqlen negative or too large";
    case FA_ERR_UNSUPPORTED_HEAD_DIM: return "FA_ERR_UNSUPPORTED_HEAD_DIM: head_dim must be 64 or 128";
    case FA_ERR_BAD_DTYPE: return "FA_ERR_BAD_DTYPE: dtype must be FA_F16 or FA_BF16";
    case FA_ERR_BAD_WINDOW: return "FA_ERR_BAD_WINDOW: window bounds must be >= -1";
    case FA_ERR_MISALIGNED: return "FA_ERR_MISALIGNED: pointers must be 16-byte aligned";
    case FA_ERR_BAD_SCALE: return "FA_ERR_BAD_SCALE: softmax_scale must be finite";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: backward workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: an output buffer is also an input buffer";
    case FA_ERR_BAD_STAGES: return "FA_ERR_BAD_STAGES: stage mask empty or unknown bits set";
    case FA_ERR_BAD_DROPOUT: return "FA_ERR_BAD_DROPOUT: dropout_p must be in [0, 1)";
    case FA_ERR_TOO_LARGE:
      return "FA_ERR_TOO_LARGE: the shape needs more statistics than fa_bwd_noalloc's static "
             "scratch holds (FA_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown fa_status";
}

const char* fa_last_error_detail(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// A packed batch ([H, total, d] arrays, per-sequence offsets): the shape checks of its rows
// per head (total) besides those of the longest sequence (seqlen).  Sets *empty as
// check_common does.
fa_status check_packed(int heads, int total, int head_dim, bool* empty) {
  if (total < 0) return FA_ERR_BAD_SHAPE;
  if ((long)total * head_dim >= kMaxRowElems) return FA_ERR_BAD_SHAPE;
  if ((long)heads * total >= kMaxRows) return FA_ERR_BAD_SHAPE;
  if (total == 0) *empty = true;
  return FA_OK;
}

// `seqlens` is the per-sequence lengths (varlen) or, with `packed`, the offsets cu[B + 1].
fa_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int* seqlens, bool varlen, int batch, int heads, int seqlen, int head_dim,
                   fa_dtype dtype, float softmax_scale, int causal, int window_left,
                   int window_right, void* stream, bool packed = false, int total = 0) {
  g_last_error.clear();
  bool empty = false;
  fa_status st = check_common(batch, heads, seqlen, head_dim, dtype, softmax_scale, window_left,
                              window_right, &empty);
  if (st != FA_OK) return st;
  if (packed && (st = check_packed(heads, total, head_dim, &empty)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || (varlen && !seqlens)) return FA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && !aligned16(lse)) || (reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0)
    return FA_ERR_MISALIGNED;
  if (o == q || o == k || o == v || (const void*)lse == q || (const void*)lse == k ||
      (const void*)lse == v || (void*)lse == o)
    return FA_ERR_ALIAS;
  if (seqlens && ((const void*)seqlens == o || (const void*)seqlens == lse)) return FA_ERR_ALIAS;

  fa::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.seqlens = packed ? nullptr : seqlens;
  p.cu = packed ? seqlens : nullptr;
  p.total = total;
  p.B = batch;
  p.H = heads;
  p.N = seqlen;
  p.D = head_dim;
  p.bf16 = dtype == FA_BF16;
  p.scale = softmax_scale;
  p.causal = causal != 0;
  p.window_left = window_left;
  p.window_right = window_right;
  return hip_status(fa::launch_fwd(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                 int heads, int seqlen, int head_dim, fa_dtype dtype, float softmax_scale,
                 int causal, int window_left, int window_right, void* stream) {
  return fwd_impl(q, k, v, o, lse, nullptr, false, batch, heads, seqlen, head_dim, dtype,
                  softmax_scale, causal, window_left, window_right, stream);
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* seqlens, int batch, int heads, int seqlen, int head_dim,
                        fa_dtype dtype, float softmax_scale, int causal, int window_left,
                        int window_right, void* stream) {
  return fwd_impl(q, k, v, o, lse, seqlens, true, batch, heads, seqlen, head_dim, dtype,
                  softmax_scale, causal, window_left, window_right, stream);
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                     int batch, int heads, int seqlen, int head_dim, fa_dtype out_dtype,
                     float softmax_scale, float q_descale, float k_descale, float v_descale,
                     int causal, int window_left, int window_right, void* stream) {
  g_last_error.clear();
  bool empty = false;
  fa_status st = check_common(batch, heads, seqlen, head_dim, out_dtype, softmax_scale,
                              window_left, window_right, &empty);
  if (st != FA_OK) return st;
  for (float x : {q_descale, k_descale, v_descale})
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_BAD_SCALE;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o) return FA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && !aligned16(lse)))
    return FA_ERR_MISALIGNED;
  if (o == q || o == k || o == v || (const void*)lse == q || (const void*)lse == k ||
      (const void*)lse == v || (void*)lse == o)
    return FA_ERR_ALIAS;
  fa::Fp8FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = batch;
  p.H = heads;
  p.N = seqlen;
  p.D = head_dim;
  p.out_bf16 = out_dtype == FA_BF16;
  p.scale = softmax_scale;
  p.q_descale = q_descale;
  p.k_descale = k_descale;
  p.v_descale = v_descale;
  p.causal = causal != 0;
  p.window_left = window_left;
  p.window_right = window_right;
  return hip_status(fa::launch_fwd_fp8(p, static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_packed(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens, int batch, int heads, int total, int max_seqlen,
                        int head_dim, fa_dtype dtype, float softmax_scale, int causal,
                        int window_left, int window_right, void* stream) {
  return fwd_impl(q, k, v, o, lse, cu_seqlens, true, batch, heads, max_seqlen, head_dim, dtype,
                  softmax_scale, causal, window_left, window_right, stream, /*packed=*/true,
                  total);
}

size_t fa_bwd_workspace_size(int batch, int heads, int seqlen, int head_dim) {
  bool empty = false;
  if (check_common(batch, heads, seqlen, head_dim, FA_BF16, 1.f, -1, -1, &empty) != FA_OK)
    return 0;
  if (empty) return 0;
  return (size_t)batch * heads * fa::stat_blocks(seqlen) * 2 * fa::kStatRows * sizeof(float);
}

}  // extern "C"

namespace {

fa_status bwd_impl(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes, const int* seqlens, bool varlen,
                   int batch, int heads, int seqlen, int head_dim, fa_dtype dtype,
                   float softmax_scale, int causal, int window_left, int window_right,
                   unsigned stages, void* stream, bool noalloc = false, bool packed = false,
                   int total = 0) {
  g_last_error.clear();
  bool empty = false;
  if (stages == 0 || (stages & ~(unsigned)FA_BWD_ALL) != 0) return FA_ERR_BAD_STAGES;
  fa_status st = check_common(batch, heads, seqlen, head_dim, dtype, softmax_scale, window_left,
                              window_right, &empty);
  if (st != FA_OK) return st;
  if (packed && (st = check_packed(heads, total, head_dim, &empty)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || (varlen && !seqlens))
    return FA_ERR_NULL_PTR;
  if ((reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0) return FA_ERR_MISALIGNED;
  const size_t need = fa_bwd_workspace_size(batch, heads, seqlen, head_dim);
  if (noalloc) {   // the static scratch replaces the workspace (it aliases no caller buffer)
    if (need > kScratchBytes) return FA_ERR_TOO_LARGE;
  } else if (!workspace || workspace_bytes < need) {
    return FA_ERR_WORKSPACE;
  }
  const void* ins[] = {q, k, v, o, dout, lse, workspace};
  void* outs[] = {dq, dk, dv};
  for (const void* p : ins)
    if (!aligned16(p)) return FA_ERR_MISALIGNED;
  for (const void* p : outs)
    if (!aligned16(p)) return FA_ERR_MISALIGNED;
  for (void* out : outs) {
    for (const void* in : ins)
      if (out == in) return FA_ERR_ALIAS;
  }
  if (dq == dk || dq == dv || dk == dv) return FA_ERR_ALIAS;
  if (seqlens && ((const void*)seqlens == dq || (const void*)seqlens == dk ||
                  (const void*)seqlens == dv || (const void*)seqlens == workspace))
    return FA_ERR_ALIAS;

  fa::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.stats = static_cast<float*>(workspace);
  p.seqlens = packed ? nullptr : seqlens;
  p.cu = packed ? seqlens : nullptr;
  p.total = total;
  p.B = batch;
  p.H = heads;
  p.N = seqlen;
  p.D = head_dim;
  p.bf16 = dtype == FA_BF16;
  p.scale = softmax_scale;
  p.causal = causal != 0;
  p.window_left = window_left;
  p.window_right = window_right;
  if (noalloc) {   // validated: only now touch the device
    p.stats = static_cast<float*>(scratch_of_current_device());
    if (p.stats == nullptr) return FA_ERR_HIP;
  }
  return hip_status(fa::launch_bwd(p, stages, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

fa_status fa_bwd_stages(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int batch, int heads, int seqlen,
                        int head_dim, fa_dtype dtype, float softmax_scale, int causal,
                        int window_left, int window_right, unsigned stages, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, nullptr, false,
                  batch, heads, seqlen, head_dim, dtype, softmax_scale, causal, window_left,
                  window_right, stages, stream);
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, const int* seqlens, int batch,
                        int heads, int seqlen, int head_dim, fa_dtype dtype, float softmax_scale,
                        int causal, int window_left, int window_right, unsigned stages,
                        void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, seqlens, true,
                  batch, heads, seqlen, head_dim, dtype, softmax_scale, causal, window_left,
                  window_right, stages, stream);
}

fa_status fa_bwd_packed(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, const int* cu_seqlens, int batch,
                        int heads, int total, int max_seqlen, int head_dim, fa_dtype dtype,
                        float softmax_scale, int causal, int window_left, int window_right,
                        unsigned stages, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, cu_seqlens, true,
                  batch, heads, max_seqlen, head_dim, dtype, softmax_scale, causal, window_left,
                  window_right, stages, stream, /*noalloc=*/false, /*packed=*/true, total);
}

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int batch, int heads, int seqlen, int head_dim, fa_dtype dtype,
                         float softmax_scale, int causal, int window_left, int window_right,
                         void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, nullptr, 0, nullptr, false, batch, heads,
                  seqlen, head_dim, dtype, softmax_scale, causal, window_left, window_right,
                  FA_BWD_ALL, stream, /*noalloc=*/true);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int batch, int heads, int seqlen, int head_dim,
                 fa_dtype dtype, float softmax_scale, int causal, int window_left,
                 int window_right, void* stream) {
  return fa_bwd_stages(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, batch,
                       heads, seqlen, head_dim, dtype, softmax_scale, causal, window_left,
                       window_right, FA_BWD_ALL, stream);
}

}  // extern "C"

namespace {

// Dense [B, H, rows, d] strides in elements.
fa::Strides dense_strides(int H, int rows, int d) {
  return fa::Strides{(long long)H * rows * d, (long long)rows * d, (long long)d};
}

// Dropout parameters as the kernels take them: the keep threshold floor(p 2^16) on 16-bit
// draws and the factor of kept weights, the inverse of the keep probability
// (2^16 - threshold) / 2^16, so that the expected weight is the undropped one (exactly 1
// without dropout).
bool dropout_from(float p, unsigned long long seed, unsigned offset, fa::Dropout* d) {
  if (!(p >= 0.f && p < 1.f)) return false;   // also rejects NaN
  d->seed_lo = (unsigned)(seed & 0xffffffffull);
  d->seed_hi = (unsigned)(seed >> 32);
  d->offset = offset;
  d->threshold = (unsigned)std::floor((double)p * 65536.0);
  d->scale = (float)(65536.0 / (double)(65536u - d->threshold));
  return true;
}

bool same_strides(const fa::Strides& a, const fa::Strides& b) {
  return a.b == b.b && a.h == b.h && a.r == b.r;
}

bool strides_ok(const fa::Strides& s, int rows) {
  if (s.b < 0 || s.h < 0 || s.r < 0) return false;
  if (s.b % 8 != 0 || s.h % 8 != 0 || s.r % 8 != 0) return false;
  // 32-bit byte offsets of rows (the kernels read up to 256 rows past the end as zeros)
  return ((long long)rows + 256) * s.r * 2 < (1LL << 31);
}

}  // namespace

extern "C" {

size_t fa_fwd_kv_workspace_size(int batch, int heads, int seqlen_q, int seqlen_k, int head_dim) {
  bool e1 = false, e2 = false;
  if (check_common(batch, heads, seqlen_q, head_dim, FA_BF16, 1.f, -1, -1, &e1) != FA_OK ||
      check_common(batch, heads, seqlen_k, head_dim, FA_BF16, 1.f, -1, -1, &e2) != FA_OK)
    return 0;
  if (batch == 0 || heads == 0 || seqlen_q == 0) return 0;
  // enough for either plan (with and without dropout)
  return std::max(fa::kv_plan(batch, heads, seqlen_q, seqlen_k, head_dim, false).ws_bytes,
                  fa::kv_plan(batch, heads, seqlen_q, seqlen_k, head_dim, true).ws_bytes);
}

fa_status fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                    const fa_strides* strides, int batch, int heads, int seqlen_q, int seqlen_k,
                    int head_dim, fa_dtype dtype, float softmax_scale, int causal,
                    int window_left, int window_right, const float* alibi_slopes,
                    const unsigned char* block_mask, const unsigned char* key_padding_mask,
                    float dropout_p, unsigned long long dropout_seed, unsigned dropout_offset,
                    void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  bool empty_q = false, empty_k = false;
  fa_status st = check_common(batch, heads, seqlen_q, head_dim, dtype, softmax_scale,
                              window_left, window_right, &empty_q);
  if (st != FA_OK) return st;
  st = check_common(batch, heads, seqlen_k, head_dim, dtype, softmax_scale, window_left,
                    window_right, &empty_k);
  if (st != FA_OK) return st;
  if (batch == 0 || heads == 0 || seqlen_q == 0) return FA_OK;
  const bool has_keys = seqlen_k > 0;
  if (!q || !o || (has_keys && (!k || !v))) return FA_ERR_NULL_PTR;

  fa::KvParams p;
  if (strides) {
    p.sq = fa::Strides{strides[0].batch, strides[0].head, strides[0].row};
    p.sk = fa::Strides{strides[1].batch, strides[1].head, strides[1].row};
    p.sv = fa::Strides{strides[2].batch, strides[2].head, strides[2].row};
    p.so = fa::Strides{strides[3].batch, strides[3].head, strides[3].row};
  } else {
    p.sq = p.so = dense_strides(heads, seqlen_q, head_dim);
    p.sk = p.sv = dense_strides(heads, seqlen_k, head_dim);
  }
  if (!strides_ok(p.sq, seqlen_q) || !strides_ok(p.so, seqlen_q) || !strides_ok(p.sk, seqlen_k) ||
      !strides_ok(p.sv, seqlen_k))
    return FA_ERR_BAD_SHAPE;

  fa::Dropout drop;
  if (!dropout_from(dropout_p, dropout_seed, dropout_offset, &drop)) return FA_ERR_BAD_DROPOUT;
  const fa::KvPlan plan = fa::kv_plan(batch, heads, seqlen_q, seqlen_k, head_dim,
                                      drop.scale != 1.f);
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes)) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(o) || (k && !aligned16(k)) || (v && !aligned16(v)) ||
      (lse && !aligned16(lse)) || (plan.ws_bytes > 0 && !aligned16(workspace)))
    return FA_ERR_MISALIGNED;
  const void* ins[] = {q, k, v};
  const void* outs[] = {o, lse, plan.ws_bytes > 0 ? workspace : nullptr};
  for (const void* out : outs) {
    if (!out) continue;
    for (const void* in : ins)
      if (out == in) return FA_ERR_ALIAS;
  }
  if ((lse && (const void*)lse == o) ||
      (outs[2] && ((const void*)outs[2] == o || (const void*)outs[2] == lse)))
    return FA_ERR_ALIAS;
  if ((reinterpret_cast<uintptr_t>(alibi_slopes) & 3u) != 0) return FA_ERR_MISALIGNED;
  for (const void* out : outs)
    if ((alibi_slopes && out == (const void*)alibi_slopes) ||
        (block_mask && out == (const void*)block_mask) ||
        (key_padding_mask && out == (const void*)key_padding_mask))
      return FA_ERR_ALIAS;

  // Plain self-attention (equal lengths, dense operands, nothing extra) takes the kernels of
  // fa_fwd, which compute the same function.
  const fa::Strides dq_ = dense_strides(heads, seqlen_q, head_dim);
  if (seqlen_q == seqlen_k && seqlen_q > fa::kDecodeMaxQ && !alibi_slopes && !block_mask &&
      !key_padding_mask && drop.scale == 1.f && same_strides(p.sq, dq_) && same_strides(p.sk, dq_) &&
      same_strides(p.sv, dq_) && same_strides(p.so, dq_)) {
    fa::FwdParams f;
    f.q = q;
    f.k = k;
    f.v = v;
    f.o = o;
    f.lse = lse;
    f.B = batch;
    f.H = heads;
    f.N = seqlen_q;
    f.D = head_dim;
    f.bf16 = dtype == FA_BF16;
    f.scale = softmax_scale;
    f.causal = causal != 0;
    f.window_left = window_left;
    f.window_right = window_right;
    return hip_status(fa::launch_fwd(f, static_cast<hipStream_t>(stream)));
  }
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.ws = plan.ws_bytes > 0 ? static_cast<float*>(workspace) : nullptr;
  p.slopes = alibi_slopes;
  p.drop = drop;
  p.blocks = block_mask;
  p.kpm = has_keys ? key_padding_mask : nullptr;
  p.B = batch;
  p.H = heads;
  p.Nq = seqlen_q;
  p.Nk = seqlen_k;
  p.D = head_dim;
  p.bf16 = dtype == FA_BF16;
  p.scale = softmax_scale;
  p.causal = causal != 0;
  p.window_left = window_left;
  p.window_right = window_right;
  return hip_status(fa::launch_fwd_kv(p, plan, static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_kv_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                        const fa_strides* strides, int batch, int heads, int seqlen_q,
                        int seqlen_k, int head_dim, fa_dtype dtype, float softmax_scale,
                        float k_descale, float v_descale, int causal, int window_left,
                        int window_right, const unsigned char* key_padding_mask, void* workspace,
                        size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  bool empty_q = false, empty_k = false;
  fa_status st = check_common(batch, heads, seqlen_q, head_dim, dtype, softmax_scale,
                              window_left, window_right, &empty_q);
  if (st != FA_OK) return st;
  st = check_common(batch, heads, seqlen_k, head_dim, dtype, softmax_scale, window_left,
                    window_right, &empty_k);
  if (st != FA_OK) return st;
  if (seqlen_q > fa::kDecodeMaxQ) return FA_ERR_BAD_SHAPE;
  if (!(std::isfinite(k_descale) && k_descale > 0.f && std::isfinite(v_descale) && v_descale > 0.f))
    return FA_ERR_BAD_SCALE;
  if (batch == 0 || heads == 0 || seqlen_q == 0) return FA_OK;
  const bool has_keys = seqlen_k > 0;
  if (!q || !o || (has_keys && (!k || !v))) return FA_ERR_NULL_PTR;

  fa::KvParams p;
  if (strides) {
    p.sq = fa::Strides{strides[0].batch, strides[0].head, strides[0].row};
    p.sk = fa::Strides{strides[1].batch, strides[1].head, strides[1].row};
    p.sv = fa::Strides{strides[2].batch, strides[2].head, strides[2].row};
    p.so = fa::Strides{strides[3].batch, strides[3].head, strides[3].row};
  } else {
    p.sq = p.so = dense_strides(heads, seqlen_q, head_dim);
    p.sk = p.sv = dense_strides(heads, seqlen_k, head_dim);
  }
  // the 16-bit bound also covers the one-byte keys and values
  if (!strides_ok(p.sq, seqlen_q) || !strides_ok(p.so, seqlen_q) || !strides_ok(p.sk, seqlen_k) ||
      !strides_ok(p.sv, seqlen_k))
    return FA_ERR_BAD_SHAPE;
  const fa::KvPlan plan = fa::kv_plan(batch, heads, seqlen_q, seqlen_k, head_dim, false, true);
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes)) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(o) || (k && !aligned16(k)) || (v && !aligned16(v)) ||
      (lse && !aligned16(lse)) || (plan.ws_bytes > 0 && !aligned16(workspace)))
    return FA_ERR_MISALIGNED;
  const void* ins[] = {q, k, v};
  const void* outs[] = {o, lse, plan.ws_bytes > 0 ? workspace : nullptr};
  for (const void* out : outs) {
    if (!out) continue;
    for (const void* in : ins)
      if (out == in) return FA_ERR_ALIAS;
  }
  if ((lse && (const void*)lse == o) ||
      (outs[2] && ((const void*)outs[2] == o || (const void*)outs[2] == lse)))
    return FA_ERR_ALIAS;
  for (const void* out : outs)
    if (key_padding_mask && out == (const void*)key_padding_mask) return FA_ERR_ALIAS;

  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.ws = plan.ws_bytes > 0 ? static_cast<float*>(workspace) : nullptr;
  p.kpm = has_keys ? key_padding_mask : nullptr;
  p.B = batch;
  p.H = heads;
  p.Nq = seqlen_q;
  p.Nk = seqlen_k;
  p.D = head_dim;
  p.bf16 = dtype == FA_BF16;
  p.fp8 = true;
  p.k_descale = k_descale;
  p.v_descale = v_descale;
  p.scale = softmax_scale;
  p.causal = causal != 0;
  p.window_left = window_left;
  p.window_right = window_right;
  return hip_status(fa::launch_fwd_kv(p, plan, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

extern "C" {

fa_status fa_bwd_kv(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, const fa_strides* strides,
                    void* workspace, size_t workspace_bytes, int batch, int heads, int seqlen_q,
                    int seqlen_k, int head_dim, fa_dtype dtype, float softmax_scale, int causal,
                    int window_left, int window_right, const float* alibi_slopes,
                    const unsigned char* block_mask, const unsigned char* key_padding_mask,
                    float dropout_p, unsigned long long dropout_seed, unsigned dropout_offset,
                    void* stream) {
  g_last_error.clear();
  bool empty_q = false, empty_k = false;
  fa_status st = check_common(batch, heads, seqlen_q, head_dim, dtype, softmax_scale,
                              window_left, window_right, &empty_q);
  if (st != FA_OK) return st;
  st = check_common(batch, heads, seqlen_k, head_dim, dtype, softmax_scale, window_left,
                    window_right, &empty_k);
  if (st != FA_OK) return st;
  if (batch == 0 || heads == 0 || (seqlen_q == 0 && seqlen_k == 0)) return FA_OK;
  const bool has_q = seqlen_q > 0, has_k = seqlen_k > 0;
  if ((has_q && (!q || !o || !dout || !lse || !dq)) || (has_k && (!k || !v || !dk || !dv)))
    return FA_ERR_NULL_PTR;

  fa::BwdKvParams p;
  if (strides) {
    fa::Strides* dst[] = {&p.sq, &p.sk, &p.sv, &p.so, &p.sg, &p.sdq, &p.sdk, &p.sdv};
    for (int i = 0; i < 8; ++i) *dst[i] = fa::Strides{strides[i].batch, strides[i].head, strides[i].row};
  } else {
    p.sq = p.so = p.sg = p.sdq = dense_strides(heads, seqlen_q, head_dim);
    p.sk = p.sv = p.sdk = p.sdv = dense_strides(heads, seqlen_k, head_dim);
  }
  const fa::Strides* qs[] = {&p.sq, &p.so, &p.sg, &p.sdq};
  const fa::Strides* ks[] = {&p.sk, &p.sv, &p.sdk, &p.sdv};
  for (const fa::Strides* x : qs)
    if (!strides_ok(*x, seqlen_q)) return FA_ERR_BAD_SHAPE;
  for (const fa::Strides* x : ks)
    if (!strides_ok(*x, seqlen_k)) return FA_ERR_BAD_SHAPE;

  const size_t need = has_q ? fa_bwd_workspace_size(batch, heads, seqlen_q, head_dim) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  const void* ins[] = {q, k, v, o, dout, lse, need > 0 ? workspace : nullptr};
  void* outs[] = {dq, dk, dv};
  for (const void* x : ins)
    if (x && !aligned16(x)) return FA_ERR_MISALIGNED;
  for (const void* x : outs)
    if (x && !aligned16(x)) return FA_ERR_MISALIGNED;
  for (void* out : outs) {
    if (!out) continue;
    for (const void* in : ins)
      if (in && out == in) return FA_ERR_ALIAS;
  }
  if ((dq && (dq == dk || dq == dv)) || (dk && dk == dv)) return FA_ERR_ALIAS;
  if ((reinterpret_cast<uintptr_t>(alibi_slopes) & 3u) != 0) return FA_ERR_MISALIGNED;
  for (void* out : outs)
    if ((alibi_slopes && out == (const void*)alibi_slopes) ||
        (block_mask && out == (const void*)block_mask) ||
        (key_padding_mask && out == (const void*)key_padding_mask))
      return FA_ERR_ALIAS;

  // Plain self-attention takes the kernels of fa_bwd (the forward took those of fa_fwd).
  {
    const fa::Strides d_ = dense_strides(heads, seqlen_q, head_dim);
    bool dense = seqlen_q == seqlen_k && seqlen_q > fa::kDecodeMaxQ;
    const fa::Strides* all[] = {&p.sq, &p.sk, &p.sv, &p.so, &p.sg, &p.sdq, &p.sdk, &p.sdv};
    for (const fa::Strides* x : all) dense = dense && same_strides(*x, d_);
    if (dense && !alibi_slopes && !block_mask && !key_padding_mask && dropout_p == 0.f) {
      fa::BwdParams b;
      b.q = q;
      b.k = k;
      b.v = v;
      b.o = o;
      b.dout = dout;
      b.lse = lse;
      b.dq = dq;
      b.dk = dk;
      b.dv = dv;
      b.stats = static_cast<float*>(workspace);
      b.B = batch;
      b.H = heads;
      b.N = seqlen_q;
      b.D = head_dim;
      b.bf16 = dtype == FA_BF16;
      b.scale = softmax_scale;
      b.causal = causal != 0;
      b.window_left = window_left;
      b.window_right = window_right;
      return hip_status(fa::launch_bwd(b, fa::kBwdAll, static_cast<hipStream_t>(stream)));
    }
  }
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.stats = static_cast<float*>(workspace);
  p.slopes = alibi_slopes;
  p.blocks = block_mask;
  p.kpm = has_k ? key_padding_mask : nullptr;
  if (!dropout_from(dropout_p, dropout_seed, dropout_offset, &p.drop)) return FA_ERR_BAD_DROPOUT;
  p.B = batch;
  p.H = heads;
  p.Nq = seqlen_q;
  p.Nk = seqlen_k;
  p.D = head_dim;
  p.bf16 = dtype == FA_BF16;
  p.scale = softmax_scale;
  p.causal = causal != 0;
  p.window_left = window_left;
  p.window_right = window_right;
  return hip_status(fa::launch_bwd_kv(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
