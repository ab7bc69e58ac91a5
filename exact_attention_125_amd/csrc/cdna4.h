// Device-side building blocks for gfx950 (CDNA4): vector types, MFMA wrappers, buffer
// loads, the LDS tile layout and cross-lane helpers.  Shared by the forward and backward
// kernels.
//
// Lane layouts used throughout (wave64, verified on the device with integer matrices):
//   v_mfma_f32_32x32x16_{bf16,f16}:  C[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[m = l%32][k = 8*(l/32) + e], e = 0..7   (one 16-byte register quad)
//     B: lane l holds B[k = 8*(l/32) + e][n = l%32]
//     C: lane l holds C[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32], i = 0..15
//   ds_read_b64_tr_b16: inside each 16-lane group, the 16 lanes' 8-byte reads form four
//     rows of 16 elements (lanes 4r..4r+3 supply row r); lane t of the group receives
//     element t of rows 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------- compile-time loop
// f(std::integral_constant<int, i>) for i = 0 .. N-1, for bodies that need i as a constant.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// ---------------------------------------------------------------------------- MFMA
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32x32x16(i16x8 a, i16x8 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// The same product issued as inline assembly with the accumulator, or the B operand, held
// in accumulation registers (AGPRs).  A kernel whose working set needs both register files
// uses these: the compiler places every builtin MFMA of a kernel in one form.  The compiler
// does not see them as matrix instructions, so their callers keep register dependencies
// apart themselves: no VALU write of an operand within a few wait states before the
// product, no other access to its result within kMfmaResultWait wait states after it (back
// to back accumulation into the same registers is resolved by the hardware).
constexpr int kMfmaResultWait = 20;   // wait states, a margin over what a 32x32x16 product needs

// acc (AGPRs) += a * b
template <bool BF16>
__device__ __forceinline__ void mfma_agpr_acc(f32x16& acc, const i16x8& a, const i16x8& b) {
  if constexpr (BF16)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// d (VGPRs) = a * b_agpr
template <bool BF16>
__device__ __forceinline__ void mfma_bagpr_first(f32x16& d, const i16x8& a, const i16x8& b) {
  if constexpr (BF16)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
// d (VGPRs) = a * b_agpr + c
template <bool BF16>
__device__ __forceinline__ void mfma_bagpr_init(f32x16& d, const i16x8& a, const i16x8& b,
                                                const f32x16& c) {
  if constexpr (BF16)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
}
// d (VGPRs) += a * b_agpr
template <bool BF16>
__device__ __forceinline__ void mfma_bagpr_acc(f32x16& d, const i16x8& a, const i16x8& b) {
  if constexpr (BF16)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}

// Two fp32 values -> two 16-bit values of the input type, round to nearest even.
template <bool BF16>
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
  if constexpr (BF16) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(unsigned, r);
  } else {
    f16x2 r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(unsigned, r);
  }
}

template <bool BF16>
__device__ __forceinline__ float to_float(unsigned short bits) {
  if constexpr (BF16) {
    return __uint_as_float(((unsigned)bits) << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, bits);
  }
}

// delta = rowsum(dO * O) of a row, in one order for every kernel that forms it: each 16-byte
// chunk (8 elements) is summed from zero one element pair (32-bit word) at a time by a packed
// dot product (the pair's two products, each exact in fp32, added to the running sum), then
// the chunk sums pairwise, neighbours first (((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7))
// ...), so the results agree bit for bit whichever kernel computes them.
template <bool BF16>
__device__ __forceinline__ float delta_chunk(const u32x4& o, const u32x4& g) {
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // (the words are copied out first: a bit cast of a vector element itself reads element 0)
    const unsigned ow = o[w], gw = g[w];
    if constexpr (BF16)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ow), __builtin_bit_cast(bf16x2, gw), acc,
                                            false);
    else
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, ow), __builtin_bit_cast(f16x2, gw), acc, false);
  }
  return acc;
}

// ---------------------------------------------------------------------------- buffer loads
// Raw buffer resource over [base, base + bytes).  Loads past the end return zeros, which
// is how tails of the sequence are read without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// ---------------------------------------------------------------------------- async copy
// 16 bytes per lane from a buffer resource straight into LDS, without passing through
// registers: lane l of the wave writes [lds + 16 l, lds + 16 l + 16).  `lds` must be the
// same in every lane of the wave.  Out-of-range offsets write zeros and touch no memory.
// The copy is counted by vmcnt; the consumer waits with wait_vmcnt and a barrier.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, char FA_LDS* lds,
                                                  int byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void FA_LDS*)lds, 16, byte_off, 0, 0, 0);
}

// s_waitcnt immediates (vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}
// The same wait as a scheduling fence: nothing is moved across it.  Values read with
// lds_read_tr_nowait look available to the compiler right after the read is issued, so
// their consumers must be kept behind the wait explicitly.
__device__ __forceinline__ void wait_lgkmcnt0_fence() {
  __builtin_amdgcn_sched_barrier(0);
  wait_lgkmcnt0();
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that the compiler neither reorders work across nor pads with waits of
// its own: callers state the waits they need (wait_vmcnt / wait_lgkmcnt0) before it.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------- LDS tiles
// A K or V tile is stored row-major, one row per key, D 16-bit elements per row, split in
// 16-byte chunks.  The chunk index is XOR-swizzled with a function of the row so that the
// three access patterns (16-byte row writes, 16-byte MFMA operand reads of 16 rows at one
// chunk, and 8-byte transposing reads of 4 rows x 4 chunks) spread over all banks.
template <int D>
__device__ __forceinline__ int chunk_swizzle(int row) {
  if constexpr (D == 64) {
    int x = (row >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
  } else {
    int x = row & 15;
    return ((x & 3) << 2) | (x >> 2);
  }
}

template <int D>
__device__ __forceinline__ int tile_offset(int row, int chunk) {  // bytes
  return row * (D * 2) + ((chunk ^ chunk_swizzle<D>(row)) << 4);
}

__device__ __forceinline__ u32x4 lds_read16(const char FA_LDS* base, int off) {
  return *reinterpret_cast<const u32x4 FA_LDS*>(base + off);
}

__device__ __forceinline__ void lds_write16(char FA_LDS* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4 FA_LDS*>(base + off) = v;
}

__device__ __forceinline__ i16x4 lds_read_tr(const char FA_LDS* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<i16x4 FA_LDS*>(const_cast<char FA_LDS*>(base) + off));
}

// The same transposing read issued as inline assembly, for kernels that manage LDS waits
// themselves: the compiler does not see it as an LDS access, so it neither waits for
// outstanding global->LDS copies before it (it would wait for all of them) nor waits for its
// result.  The caller must s_waitcnt lgkmcnt(0) before using the value.  `addr` is an LDS
// byte address, OFF an immediate byte offset.
template <int OFF>
__device__ __forceinline__ i16x4 lds_read_tr_nowait(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  i16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// A 16-byte LDS read issued the same way (no compiler-inserted waits before or after it).
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16_nowait(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// s_waitcnt lgkmcnt(N) as a scheduling fence: at most N LDS reads still in flight.  LDS reads
// complete in issue order, so this waits for every read but the N latest.
template <int N>
__device__ __forceinline__ void wait_lgkmcnt_fence() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (N << 8));
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ unsigned lds_addr(const char FA_LDS* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>(p));
}

// Empty statements that make a value be computed before this point (the compiler may not
// sink it past a barrier into the phase that uses it).  They emit no instruction.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(unsigned& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(f32x16& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(i16x4& x) { asm volatile("" : "+v"(x)); }
// Moves x into accumulation registers (AGPRs) at this point; used for values that only
// register-placed MFMAs read or write afterwards.
__device__ __forceinline__ void in_agpr(i16x8& x) { asm volatile("" : "+a"(x)); }
__device__ __forceinline__ void in_agpr(f32x16& x) { asm volatile("" : "+a"(x)); }
// Wait states between register-placed MFMAs and other accesses to their registers:
// kMfmaResultWait after a product before its result is read, a few before a product reads a
// register a VALU instruction wrote.
__device__ __forceinline__ void mfma_result_wait() { asm volatile("s_nop 15\n\ts_nop 7" ::: "memory"); }
__device__ __forceinline__ void mfma_operand_wait() { asm volatile("s_nop 7" ::: "memory"); }
// An empty statement the compiler may not speculate: placed in a branch's body, it keeps the
// branch (the body is not turned into selects that run on every path).
__device__ __forceinline__ void keep_branch() { asm volatile("" ::: "memory"); }
// Keeps x in its registers, unchanged, up to this point (its registers are not reused before).
__device__ __forceinline__ void keep(const f32x16& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void keep(const f32x4& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void keep(const u32x4& x) { asm volatile("" ::"v"(x)); }

// ---------------------------------------------------------------------------- cross-lane
// The partner of lane l is lane l ^ 32.  permlane32_swap(x, x) leaves {x[l], x[l^32]} in
// some order in every lane, so a symmetric combine of the pair is the wave-wide result.
__device__ __forceinline__ float max_with_partner(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float min_with_partner(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_with_partner(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------- dropout
// Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel
// Random Numbers: As Easy as 1, 2, 3", SC 2011): ten rounds of two 32x32 -> 64-bit products
// (multipliers 0xD2511F53, 0xCD9E8D57) mixed with the other counter words and the key, the key
// bumped by (0x9E3779B9, 0xBB67AE85) between rounds.  The key schedule is wave-uniform.
__device__ __forceinline__ void philox4x32_10(unsigned c0, unsigned c1, unsigned c2, unsigned c3,
                                              unsigned k0, unsigned k1, unsigned (&out)[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const unsigned long long p0 = (unsigned long long)0xD2511F53u * c0;
    const unsigned long long p1 = (unsigned long long)0xCD9E8D57u * c2;
    const unsigned n0 = (unsigned)(p1 >> 32) ^ c1 ^ k0;
    const unsigned n2 = (unsigned)(p0 >> 32) ^ c3 ^ k1;
    c1 = (unsigned)p1;
    c3 = (unsigned)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;   // the bump after the last round is never used
    k1 += 0xBB67AE85u;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// Dropout of attention weights: one generator call draws 16 bits for each of 2 queries x 4
// keys of one (batch, head): counter (j >> 2, i >> 1, batch * heads + head, offset), key = the
// 64-bit seed; pair (i, j) takes half-word 4 (i & 1) + (j & 3) (word t >> 1, high half when t
// is odd) and is kept when that half-word is at least floor(p 2^16).
struct Dropout {
  unsigned seed_lo, seed_hi, offset;
  unsigned threshold;   // floor(p 2^16); 0 keeps everything
  float scale;          // 2^16 / (2^16 - threshold): inverse of the keep probability
  // the call that holds the draws of queries i & ~1, i | 1 for keys j & ~3 .. j | 3
  __device__ __forceinline__ void call(int bh, int i, int j, unsigned (&o)[4]) const {
    philox4x32_10((unsigned)j >> 2, (unsigned)i >> 1, (unsigned)bh, offset, seed_lo, seed_hi, o);
  }
  // whether (i, j) is kept, from its call's words
  __device__ __forceinline__ bool keep(const unsigned (&o)[4], int i, int j) const {
    const int t = 4 * (i & 1) + (j & 3);
    const unsigned w = (t >> 1) == 0 ? o[0] : (t >> 1) == 1 ? o[1] : (t >> 1) == 2 ? o[2] : o[3];
    return ((t & 1) ? (w >> 16) : (w & 0xffffu)) >= threshold;
  }
  __device__ __forceinline__ bool keep_half(unsigned w, int high) const {
    return (high ? (w >> 16) : (w & 0xffffu)) >= threshold;
  }
  // Query-per-lane layouts (forward, dQ): lane l holds query i with i & 1 == l & 1, and keys in
  // four runs jr0 + 8 r + 0..3 (r = 0..3).  The queries 2a, 2a + 1 of lanes l, l ^ 1 share
  // every call, so each lane makes the calls of two runs and swaps words with its neighbour
  // (DPP quad_perm [1, 0, 3, 2]; every lane of the wave must be active).  out[r] = the words
  // of query i for keys jr, jr + 1 (out[r][0], low / high half) and jr + 2, jr + 3 (out[r][1]).
  __device__ __forceinline__ void runs4(int bh, int i, int jr0, unsigned (&out)[4][2]) const {
    const int par = i & 1;
    unsigned own[2][4];
    call(bh, i, jr0 + 8 * (2 * par + 0), own[0]);
    call(bh, i, jr0 + 8 * (2 * par + 1), own[1]);
    unsigned recv[2][2];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        // the neighbour's query has the other parity: send it the words of that parity
        const unsigned send = par ? own[rr][w] : own[rr][2 + w];
        recv[rr][w] = (unsigned)__builtin_amdgcn_update_dpp(0, (int)send, 0xB1, 0xF, 0xF, false);
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool mine = (r >> 1) == par;
#pragma unroll
      for (int w = 0; w < 2; ++w)
        out[r][w] = mine ? (par ? own[r & 1][2 + w] : own[r & 1][w]) : recv[r & 1][w];
    }
  }
  // Key-per-lane layout (dK/dV): lane l holds key j with j & 3 == l & 3 and, per step, queries
  // q0 + 8 g + 2 c' + 0..1 for the call index c = 2 g + c' (c = 0..7).  The four lanes of a quad
  // (keys 4a .. 4a + 3) share every call, so lane (l & 3) makes calls 2 (l & 3) and
  // 2 (l & 3) + 1 and the quad broadcasts them.  out[c] = the words of the even and the odd query
  // of call c for this lane's key (low half for even keys, high half for odd ones).
  __device__ __forceinline__ void pairs8(int bh, int q0, int j, unsigned (&out)[8][2]) const {
    const int kq = j & 3;
    unsigned own[2][4];
    call(bh, q0 + 8 * kq + 0, j, own[0]);
    call(bh, q0 + 8 * kq + 2, j, own[1]);
    static_for<8>([&](auto cc) {
      constexpr int c = decltype(cc)::value, owner = c >> 1, r = c & 1;
      constexpr int kBcast = owner | (owner << 2) | (owner << 4) | (owner << 6);   // quad_perm
      unsigned x[4];
#pragma unroll
      for (int w = 0; w < 4; ++w)
        x[w] = (unsigned)__builtin_amdgcn_update_dpp(0, (int)own[r][w], kBcast, 0xF, 0xF, false);
      out[c][0] = (kq >> 1) ? x[1] : x[0];
      out[c][1] = (kq >> 1) ? x[3] : x[2];
    });
  }
};

// ---------------------------------------------------------------------------- masks
// The 32x32 MFMA accumulator layout: element i of lane L sits in row 8 (i/4) + 4 (L/32) + i%4
// and column L % 32.  diag_lanes<KeyRows>(i) is the wave-wide lane mask of the elements i on
// or below the diagonal of a block whose rows and columns start at the same sequence
// position: row >= column when rows are queries and columns keys, column >= row when rows are
// keys and columns queries, i.e. query >= key either way.
template <bool KeyRows>
constexpr unsigned long long diag_lanes(int i) {
  unsigned long long m = 0;
  for (int lane = 0; lane < 64; ++lane) {
    const int row = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3), col = lane & 31;
    if (KeyRows ? col >= row : row >= col) m |= 1ull << lane;
  }
  return m;
}
// x in the lanes whose bit of the (wave-uniform) mask is set, 0 elsewhere: one v_cndmask with
// the mask as its scalar condition
__device__ __forceinline__ float keep_lanes(float x, unsigned long long lanes) {
  return __builtin_amdgcn_inverse_ballot_w64(lanes) ? x : 0.f;
}

// Key j is visible to query i iff (!causal || j <= i) && (wl < 0 || j >= i - wl)
// && (wr < 0 || j <= i + wr), and j < N.
struct Mask {
  int n, causal, wl, wr;
  __device__ __forceinline__ bool visible(int i, int j) const {
    bool ok = j < n;
    if (causal) ok = ok && (j <= i);
    if (wl >= 0) ok = ok && (j >= i - wl);
    if (wr >= 0) ok = ok && (j <= i + wr);
    return ok;
  }
  // Key range [lo, hi) that queries [q_first, q_last] can see at all.
  __device__ __forceinline__ void key_range(int q_first, int q_last, int& lo, int& hi) const {
    lo = wl >= 0 ? max(0, q_first - wl) : 0;
    hi = n;
    if (causal) hi = min(hi, q_last + 1);
    if (wr >= 0) hi = min(hi, q_last + wr + 1);
  }
  // Whether every (i, j) in [q_first, q_last] x [j0, j1) is visible.
  __device__ __forceinline__ bool all_visible(int q_first, int q_last, int j0, int j1) const {
    bool ok = j1 <= n;
    if (causal) ok = ok && (j1 - 1 <= q_first);
    if (wl >= 0) ok = ok && (j0 >= q_last - wl);
    if (wr >= 0) ok = ok && (j1 - 1 <= q_first + wr);
    return ok;
  }
  // Query range [lo, hi) that keys [k_first, k_last] are visible to (for key-owned passes).
  __device__ __forceinline__ void query_range(int k_first, int k_last, int& lo, int& hi) const {
    lo = 0;
    hi = n;
    if (causal) lo = max(lo, k_first);
    if (wr >= 0) lo = max(lo, k_first - wr);
    if (wl >= 0) hi = min(hi, k_last + wl + 1);
  }
};

// ---------------------------------------------------------------------------- grid order
// The hardware hands consecutive workgroup ids to the 8 XCDs in turn (id % 8), and each
// XCD has its own L2.  Map ids so that all tiles of one (batch, head) run on one XCD and
// reuse that head's K/V from the same L2, walking each head's tiles in the given order.
__device__ __forceinline__ void xcd_tile_order(int id, int n_bh, int n_tiles, int& bh, int& tile) {
  if ((n_bh & 7) == 0) {
    int xcd = id & 7;
    int slot = id >> 3;
    bh = (slot / n_tiles) * 8 + xcd;
    tile = slot % n_tiles;
  } else {
    bh = id / n_tiles;
    tile = id % n_tiles;
  }
}

}  // namespace fa
