// decode_rows.h -- the rows of one expert group found from the expert ids
// themselves, for decode-sized batches (at most 64 tokens), and the
// permutation written on the way.  Shared by the decode gate_up kernels
// (bf16 and MXFP4 weights): the grouped execution needs each expert's rows
// (aitoday "MoEs in Transformers" page, section "Expert Backend"), and at
// decode sizes the gate_up workgroups can find them with a few ballots
// instead of a separate permutation launch.
#pragma once
#include "moe_common.h"

namespace moe {
namespace {

// Rows of one expert group in the fused form: the copies s (ascending) whose
// expert id is g, found from the ids themselves.  n_slots = T*k <= 4096.
struct GroupFromIds {
  int row_begin, rows;
};
// One wave's view: ballots over the ids, 64 at a time.  `list` (LDS, >= 64
// entries) receives the group's copies in ascending order (a group has at
// most T <= 64 of them: a token picks an expert at most once).  Ids outside
// [0, E) count for no group; their copies take the first rows (the layout
// of the permutation step), so group g starts after them and after the
// copies of the groups below g.
__device__ __forceinline__ GroupFromIds group_from_ids(const int32_t* __restrict__ idx,
                                                       int n_slots, int g, int E, int* list) {
  const int lane = threadIdx.x & 63;
  const uint64_t below_lanes = (1ull << lane) - 1ull;
  int before = 0, found = 0;
  for (int s0 = 0; s0 < n_slots; s0 += 64) {
    const int s = s0 + lane;
    const bool in = s < n_slots;
    const uint32_t v = in ? (uint32_t)idx[s] : 0u;  // unsigned: ids < 0 are huge
    // copies placed before group g: ids below g, and ids outside [0, E)
    const uint64_t lt = __ballot(in && (v < (uint32_t)g || v >= (uint32_t)E));
    const uint64_t eq = __ballot(in && v == (uint32_t)g);
    if ((eq >> lane) & 1ull) {
      const int r = found + __popcll(eq & below_lanes);
      if (r < 64) list[r] = s;
    }
    before += __popcll(lt);
    found += __popcll(eq);
  }
  return GroupFromIds{before, found};
}

// Outputs of the permutation step, written by the gate_up kernel.
struct DecodePerm {
  int32_t* counts;     // [G]
  int32_t* offsets;    // [G + 1]
  int32_t* sorted;     // [T*k] sorted_slot
  int32_t* slot_pos;   // [T*k]
};

// Group g's first row and row count (every wave of the workgroup calls
// this; each finds the group itself and writes the same s_list values).
// The workgroups of column tile 0 write the permutation: wave 0 of each
// group its counts / offsets and its sorted_slot / slot_pos entries, wave 1
// of group 0 the copies whose id lies outside [0, E) (listed first, in slot
// order, with slot_pos -1).  Shared expert g - E takes every token.
__device__ __forceinline__ void decode_group_rows(const int32_t* __restrict__ topk_idx, int g,
                                                  int G, int E, int64_t T, int64_t Tk,
                                                  int tile, int wave, int* s_list,
                                                  const DecodePerm& p, int64_t* row_begin,
                                                  int64_t* rows) {
  const int lane = threadIdx.x & 63;
  if (g < E) {
    // a token picks an expert at most once, so a group has at most T <= 64 rows
    const GroupFromIds gi = group_from_ids(topk_idx, (int)Tk, g, E, s_list);
    *row_begin = gi.row_begin;
    *rows = gi.rows < 64 ? gi.rows : 64;
  } else {
    *row_begin = Tk + (int64_t)(g - E) * T;
    *rows = T;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (tile == 0 && wave == 0) {
    if (lane == 0) {
      p.counts[g] = (int32_t)*rows;
      p.offsets[g] = (int32_t)*row_begin;
      if (g == G - 1) p.offsets[G] = (int32_t)(Tk + (int64_t)(G - E) * T);
    }
    if (g < E) {
      for (int r = lane; r < *rows && r < 64; r += 64) {
        const int sl = s_list[r];
        p.sorted[*row_begin + r] = sl;
        p.slot_pos[sl] = (int32_t)(*row_begin + r);
      }
    }
  }
  if (g == 0 && tile == 0 && wave == 1) {
    const uint64_t below_lanes = (1ull << lane) - 1ull;
    int at = 0;
    for (int s0 = 0; s0 < (int)Tk; s0 += 64) {
      const int sl = s0 + lane;
      const bool drop = sl < (int)Tk && (uint32_t)topk_idx[sl] >= (uint32_t)E;
      const uint64_t m = __ballot(drop);
      if (drop) {
        p.sorted[at + __popcll(m & below_lanes)] = sl;
        p.slot_pos[sl] = -1;
      }
      at += __popcll(m);
    }
  }
}

// Token of row r (< rows) of group g, as found by decode_group_rows; grow is
// the row's index in the permuted order.
__device__ __forceinline__ int64_t decode_row_token(int g, int E, int64_t r, int64_t grow,
                                                    int64_t Tk, int64_t T, int64_t k,
                                                    const int* s_list) {
  return g < E ? (int64_t)((uint32_t)s_list[r < 64 ? r : 63] / (uint32_t)k)
               : (int64_t)((uint32_t)(grow - Tk) % (uint32_t)T);
}

}  // namespace
}  // namespace moe
