// permute.hip -- group the T*k token copies by expert: per-expert histogram,
// exclusive prefix sum, stable scatter.
//
// The grouped execution sorts the token copies by expert id so that every
// expert runs one contiguous block of rows, and the results are gathered
// back to token order afterwards (aitoday "MoEs in Transformers" page,
// section "Expert Backend", grouped_mm).  Order inside a group: ascending
// copy id s = t*k + j, which makes the permutation unique.
//
// One workgroup of 16 waves.  Wave w owns the contiguous copy range
// [w*seg, (w+1)*seg) and walks it 64 copies at a time:
//   A. rank every copy among the earlier copies of its expert in the same
//      wave range: lanes with equal expert id are found with one ballot per
//      id bit; the rank inside the 64 is a popcount of the lower peer lanes,
//      and the highest peer lane advances that expert's running count in the
//      wave's LDS histogram row (one wave's LDS operations run in program
//      order, so the next 64 see the update).  The rank is parked in slot_pos.
//   B. per expert: total over the 16 rows, block-wide exclusive scan -> offsets,
//      and each row is turned into that wave's base position for the expert.
//   C. position = base[w][e] + rank; sorted_slot[position] = s.
// Integer only: the result is exact and independent of scheduling.
//
// Ids outside [0, E) select no expert: such a copy is ranked in a bin of its
// own after all experts, so it lands in rows [valid, T*k) (inside the last
// expert's row range, since offsets[E] = T*k always; that expert's count does
// not include them) and gets slot_pos = -1, which the combine skips.  Every
// row below T*k is thus written, every index stays in bounds, and the shared
// rows always start at T*k.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxGroups = 1024;
constexpr int kBatch = 16;  // steps of 64 copies whose loads are issued together

__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int wv = lane < kWaves ? tmp[lane] : 0;
    int winc = wv;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      const int o = __shfl_up(winc, off, 64);
      if (lane >= off) winc += o;
    }
    if (lane < kWaves) tmp[kWaves + lane] = winc - wv;  // exclusive wave base
    if (lane == kWaves - 1) tmp[2 * kWaves] = winc;
  }
  __syncthreads();
  *total = tmp[2 * kWaves];
  return tmp[kWaves + wave] + inc - v;
}

__global__ __launch_bounds__(kThreads) void permute_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ slot_pos, int64_t T, int64_t k, int E, int S, int nbits) {
  __shared__ int32_t hist[kWaves][kMaxGroups + 1];  // + the bin of dropped copies
  __shared__ int32_t tmp[2 * kWaves + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t n = T * k;
  const int64_t seg = (n + kWaves - 1) / kWaves;
  const int64_t s_begin = wave * seg;
  const int64_t s_end = s_begin + seg < n ? s_begin + seg : n;
  const uint64_t lanes_below = (1ull << lane) - 1ull;

  for (int e = lane; e <= E; e += 64) hist[wave][e] = 0;

  // ---- A: rank inside the wave's range; the expert ids of kBatch steps of
  // 64 copies are loaded up front so their latency overlaps
  for (int64_t b0 = s_begin; b0 < s_end; b0 += 64 * kBatch) {
    int v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t s = b0 + 64 * u + lane;
      v[u] = s < s_end ? idx[s] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (b0 + 64 * u >= s_end) break;
      const int64_t s = b0 + 64 * u + lane;
      const bool active = s < s_end;
      // expert id; E: the dropped bin (ids outside [0, E)); E + 1: idle lane
      const int key = !active ? E + 1 : (v[u] >= 0 && v[u] < E) ? v[u] : E;
      uint64_t peers = ~0ull;
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bal = __ballot(bit);
        peers &= bit ? bal : ~bal;
      }
      const int rank = __popcll(peers & lanes_below);
      const int leader = 63 - __clzll(peers);
      int before = 0;
      if (active && lane == leader) {
        before = hist[wave][key];
        hist[wave][key] = before + __popcll(peers);
      }
      before = __shfl(before, leader, 64);
      if (active) slot_pos[s] = before + rank;
    }
  }
  __syncthreads();

  // ---- B: totals, prefix sum over the routed experts, per-wave bases; the
  // dropped bin follows the routed rows, the shared groups start at T*k
  const int g = threadIdx.x;  // expert group handled by this thread
  int total = 0;
  if (g < E) {
    for (int w = 0; w < kWaves; ++w) total += hist[w][g];
  } else if (g < E + S) {
    total = (int)T;
  }
  int valid = 0;
  const int off = block_exclusive_scan(g < E ? total : 0, tmp, &valid);
  const int Tk = (int)(T * k);
  if (g < E) {
    counts[g] = total;
    offsets[g] = off;
  } else if (g < E + S) {
    counts[g] = total;
    offsets[g] = Tk + (g - E) * (int)T;
  }
  if (g == 0) offsets[E + S] = Tk + S * (int)T;
  if (g <= E) {
    int run = g < E ? off : valid;
    for (int w = 0; w < kWaves; ++w) {
      const int c = hist[w][g];
      hist[w][g] = run;
      run += c;
    }
  }
  __syncthreads();

  // ---- C: scatter (loads batched as in A)
  for (int64_t b0 = s_begin; b0 < s_end; b0 += 64 * kBatch) {
    int v[kBatch], r[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t s = b0 + 64 * u + lane;
      v[u] = s < s_end ? idx[s] : -1;
      r[u] = s < s_end ? slot_pos[s] : 0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t s = b0 + 64 * u + lane;
      if (s >= s_end) continue;
      const bool dropped = v[u] < 0 || v[u] >= E;
      const int pos = hist[wave][dropped ? E : v[u]] + r[u];
      sorted_slot[pos] = (int32_t)s;
      slot_pos[s] = dropped ? -1 : pos;
    }
  }
}

}  // namespace

hipError_t launch_permute(const Shape& s, const int32_t* topk_idx, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos,
                          hipStream_t st) {
  int nbits = 0;
  while ((1 << nbits) <= s.E + 1) ++nbits;  // keys 0..E+1 (E: dropped, E+1: idle lane)
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kThreads), 0, st, topk_idx, counts,
                     offsets, sorted_slot, slot_pos, s.T, s.k, (int)s.E, (int)s.S,
                     nbits);
  return hipGetLastError();
}

}  // namespace moe
