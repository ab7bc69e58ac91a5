// Block-sparse masks on the tuned kernels: the list of the steps a workgroup visits.
//
// A block mask selects 64 x 64 blocks of (queries, keys).  A tuned workgroup owns NB
// consecutive 64-row blocks of one axis (its own rows: queries for the forward and dQ, keys for
// dK/dV) and streams the other axis in steps of TILE rows.  It visits the steps one of its
// blocks selects, in order, and a wave whose own block does not select a visited step sees all
// of that step's pairs hidden.  The list of visited steps is built in LDS at the start of a
// tile, from one selection word per (chunk of 64 steps, own block): a wave ballots its chunks'
// mask bytes, then every wave counts the words of the chunks before its own to place entries.
#pragma once

#include "cdna4.h"

namespace fa {

// most steps a list holds (a head's streamed axis in steps)
constexpr int kListMax = 1024;
// list slots: entries, the sentinels and reads past them up to one window of 64, the count
constexpr int kListSlots = kListMax + 64 + 8;
constexpr int kListCount = kListSlots - 1;

// LDS bytes of a list for NB own blocks: the slots, then NB selection words per chunk
template <int NB>
constexpr int block_list_bytes() {
  return 4 * kListSlots + 8 * NB * (kListMax / 64);
}

// Builds the list of the workgroup's visited steps and returns its length.  The mask of the
// head is reached from bm as bm[own block * own_stride + streamed block * str_stride]; the
// workgroup owns blocks ob0 .. ob0 + NB - 1 (those at or past n_own select nothing) and streams
// steps s_begin .. s_begin + T - 1 of TILE rows (T <= kListMax).  Entry k is the k-th visited
// step r (counted from s_begin) with bit 16 + i set when own block i selects it; NSENT entries
// 0xffff (a step past T, selected by no block) follow the last one.  Every wave of the
// workgroup calls it; it ends with a barrier.
template <int NB, int TILE, int NSENT, int WAVES>
__device__ __forceinline__ int build_block_list(int FA_LDS* list, const unsigned char* bm,
                                                long own_stride, long str_stride, int ob0, int n_own,
                                                int s_begin, int T, int lane, int wave) {
  static_assert(NB >= 1 && NB <= 4 && NSENT <= 64, "own blocks and sentinels the slots hold");
  static_assert((WAVES & (WAVES - 1)) == 0, "chunks go round the waves by a mask");
  unsigned long long FA_LDS* words = (unsigned long long FA_LDS*)(list + kListSlots);
  const int nch = (T + 63) >> 6;
  for (int ch = wave; ch < nch; ch += WAVES) {
    const int r = 64 * ch + lane;
    const long sb = r < T ? (long)(((s_begin + r) * TILE) >> 6) * str_stride : 0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const bool sel = r < T && ob0 + i < n_own && bm[(long)(ob0 + i) * own_stride + sb] != 0;
      const unsigned long long w = __ballot(sel);
      if (lane == 0) words[NB * ch + i] = w;
    }
  }
  wait_lgkmcnt0();   // (the barrier does not wait for LDS writes)
  wg_barrier();
  int total = 0;
  for (int ch = 0; ch < nch; ++ch) {
    unsigned long long w[NB], any = 0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      w[i] = words[NB * ch + i];
      any |= w[i];
    }
    if ((ch & (WAVES - 1)) == wave && ((any >> lane) & 1ull)) {
      int e = 64 * ch + lane;
#pragma unroll
      for (int i = 0; i < NB; ++i) e |= (int)((w[i] >> lane) & 1ull) << (16 + i);
      list[total + __builtin_popcountll(any & ((1ull << lane) - 1ull))] = e;
    }
    total += __builtin_popcountll(any);
  }
  if (wave == 0) {
    if (lane < NSENT) list[total + lane] = 0xffff;
    if (lane == 0) list[kListCount] = total;
  }
  wait_lgkmcnt0();
  wg_barrier();
  return __builtin_amdgcn_readfirstlane(list[kListCount]);
}

// the step of a list entry, and whether own block i selects it
__device__ __forceinline__ int entry_step(int e) { return e & 0xffff; }
__device__ __forceinline__ bool entry_selected(int e, int i) { return (e >> (16 + i)) & 1; }

}  // namespace fa
