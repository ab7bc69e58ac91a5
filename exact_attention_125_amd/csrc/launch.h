// Internal interface between the validating C-ABI layer (api.cpp) and the kernel
// launchers (fwd.hip, bwd.hip).  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // may be null
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
  float* delta;        // workspace: rowsum(dO * O), [B, H, N] fp32
  int B, H, N, D;
  bool bf16;
  float scale;
  int causal;
  int window_left;
  int window_right;
};

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);
// The 8-wave forward (256 query rows per workgroup, direct global->LDS copies, two-phase
// software pipeline), for grids that fill the chip; launch_fwd chooses between it and the
// four-wave kernel of fwd.hip.
hipError_t launch_fwd_main(const FwdParams& p, hipStream_t stream);
// Backward stages, run in this order on one stream: delta = rowsum(dO * O) into the
// workspace, then dK/dV, then dQ (both read delta).
constexpr unsigned kBwdDelta = 1u, kBwdDkDv = 2u, kBwdDq = 4u, kBwdAll = 7u;
hipError_t launch_bwd(const BwdParams& p, unsigned stages, hipStream_t stream);

}  // namespace fa
