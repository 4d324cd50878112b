// permute.hip -- group the T*k token copies by expert: per-expert histogram,
// exclusive prefix sum, stable scatter.
//
// The grouped execution sorts the token copies by expert id so that every
// expert runs one contiguous block of rows, and the results are gathered
// back to token order afterwards (aitoday "MoEs in Transformers" page,
// section "Expert Backend", grouped_mm).  Order inside a group: ascending
// copy id s = t*k + j, which makes the permutation unique.
//
// Batches below 8192 copies: one workgroup of 16 waves (larger ones: the
// multi-workgroup form further down).  Wave w owns the contiguous copy range
// [w*seg, (w+1)*seg) and walks it 64 copies at a time:
//   A. rank every copy among the earlier copies of its expert in the same
//      wave range: lanes with equal expert id are found with one ballot per
//      id bit; the rank inside the 64 is a popcount of the lower peer lanes,
//      and the highest peer lane advances that expert's running count in the
//      wave's LDS histogram row (one wave's LDS operations run in program
//      order, so the next 64 see the update).  The rank is parked in slot_pos.
//   B. per expert: total over the 16 rows, block-wide exclusive scans ->
//      offsets, and each row is turned into the rank (among all copies of
//      the expert) of that wave's first copy of it.
//   C. rank = that base + the rank inside the wave range; position = the
//      first row of the expert's kept (or dropped) copies + rank;
//      sorted_slot[position] = s.
// Integer only: the result is exact and independent of scheduling.
//
// Expert capacity (optional): every expert keeps at most `cap` copies, its
// first ones in slot order, and drops the rest (yunthe "分工的艺术" page,
// section 3.1, expert capacity; Baidu page, section 三.2, capacity-bound
// token dropping).  A copy's rank among its expert's copies is its wave
// base plus its rank inside the wave range, so the test is one compare.
//
// Dropped copies take the rows at the front, [0, D): first the copies whose
// id lies outside [0, E) (they select no expert), in slot order, then the
// copies over capacity, by expert, in slot order; their slot_pos is -1,
// which the combine skips.  Kept copies follow from offsets[0] = D, so no
// expert group contains a dropped row and offsets[E] = T*k always: every
// row below T*k is written, every index stays in bounds, and the shared
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
    int32_t* __restrict__ slot_pos, int64_t T, int64_t k, int E, int S, int nbits, int cap) {
  __shared__ int32_t hist[kWaves][kMaxGroups + 1];  // + the bin of invalid ids
  __shared__ int32_t row_kept[kMaxGroups];           // first row of expert e's kept copies
  __shared__ int32_t row_over[kMaxGroups];           // first row of its copies over capacity
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
      // expert id; E: the bin of invalid ids (outside [0, E)); E + 1: idle lane
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

  // ---- B: per expert, kept = min(copies, cap) and over = the rest; the
  // invalid ids' rows, then every expert's rows over capacity, then the kept
  // rows (prefix sum of kept); the shared groups start at T*k
  const int g = threadIdx.x;  // expert group handled by this thread
  int total = 0;
  if (g < E)
    for (int w = 0; w < kWaves; ++w) total += hist[w][g];
  int n_inv = 0;
  for (int w = 0; w < kWaves; ++w) n_inv += hist[w][E];
  const int kept = g < E ? (total < cap ? total : cap) : 0;
  int n_over = 0, n_kept = 0;
  const int over_base = n_inv + block_exclusive_scan(g < E ? total - kept : 0, tmp, &n_over);
  const int kept_off = block_exclusive_scan(kept, tmp, &n_kept);
  const int n_drop = n_inv + n_over;
  const int Tk = (int)(T * k);
  if (g < E) {
    counts[g] = kept;
    offsets[g] = n_drop + kept_off;
  } else if (g < E + S) {
    counts[g] = (int)T;
    offsets[g] = Tk + (g - E) * (int)T;
  }
  if (g == 0) offsets[E + S] = Tk + S * (int)T;
  // per wave and expert: the rank (among the expert's copies) of the wave's
  // first copy of it
  if (g < E) {
    row_kept[g] = n_drop + kept_off;
    row_over[g] = over_base;
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = hist[w][g];
      hist[w][g] = run;
      run += c;
    }
  }
  if (g == 0) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = hist[w][E];
      hist[w][E] = run;
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
      const bool valid = v[u] >= 0 && v[u] < E;
      const int rank = hist[wave][valid ? v[u] : E] + r[u];  // among the same key's copies
      const bool keep = valid && rank < cap;
      const int pos = !valid ? rank : keep ? row_kept[v[u]] + rank : row_over[v[u]] + rank - cap;
      sorted_slot[pos] = (int32_t)s;
      slot_pos[s] = keep ? pos : -1;
    }
  }
}

// ------------------------------------------------------- multi-workgroup
// For large batches (n >= kMultiMin copies) the same permutation in four
// launches, none of whose workgroups waits for another:
//   1. rank (NB workgroups of kChunk copies): each copy's rank among the
//      earlier copies of its key in the workgroup (per-wave ranks as in A,
//      plus the wave's base inside the workgroup), parked in slot_pos; the
//      workgroup's key histogram becomes row b of H.
//   2. scan (one workgroup): per key, the exclusive prefix of H's rows in
//      place; counts and offsets as in B; row NB of H gets the first row of
//      each expert's copies over capacity.
//   3. place (NB workgroups): row = the key's first row + prefix + parked
//      rank, stored in slot_pos (a dropped copy as -2 - row).
//   4. scatter: sorted_slot[row] = s, slot_pos = -1 for dropped copies.
// H, (NB + 1) x (E + 1) int32, lives in sorted_slot until step 4: steps 1-3
// write no other entry of sorted_slot, and step 4 reads no entry of H.
constexpr int kChunk = 2 * 64 * kWaves;  // copies per workgroup: 2 steps per wave
constexpr int64_t kMultiMin = 8192;

__global__ __launch_bounds__(kThreads) void permute_rank_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ slot_pos, int32_t* __restrict__ H,
    int64_t n, int E, int nbits) {
  extern __shared__ int32_t whist[];  // [kWaves][E + 1]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int E1 = E + 1;
  int32_t* hist = whist + wave * E1;
  const uint64_t lanes_below = (1ull << lane) - 1ull;
  const int64_t s0 = (int64_t)blockIdx.x * kChunk + wave * 128 + lane;
  int v[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) v[u] = s0 + 64 * u < n ? idx[s0 + 64 * u] : -1;
  for (int e = lane; e < E1; e += 64) hist[e] = 0;
  int key[2], r[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const bool active = s0 + 64 * u < n;
    // E: the bin of invalid ids; E + 1: idle lane
    key[u] = !active ? E + 1 : (v[u] >= 0 && v[u] < E) ? v[u] : E;
    uint64_t peers = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key[u] >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int leader = 63 - __clzll(peers);
    int before = 0;
    if (active && lane == leader) {
      before = hist[key[u]];
      hist[key[u]] = before + __popcll(peers);
    }
    r[u] = __shfl(before, leader, 64) + __popcll(peers & lanes_below);
  }
  __syncthreads();
  // per key: the waves' exclusive bases inside the workgroup, and its total
  for (int e = threadIdx.x; e < E1; e += kThreads) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = whist[w * E1 + e];
      whist[w * E1 + e] = run;
      run += c;
    }
    H[(int64_t)blockIdx.x * E1 + e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (s0 + 64 * u < n) slot_pos[s0 + 64 * u] = hist[key[u]] + r[u];
}

__global__ __launch_bounds__(kThreads) void permute_scan_kernel(
    int32_t* __restrict__ H, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int64_t T, int64_t k, int E, int S, int NB, int cap) {
  __shared__ int32_t part[kThreads];
  __shared__ int32_t tot[kThreads];
  __shared__ int32_t tmp[2 * kWaves + 1];
  const int tid = threadIdx.x;
  const int E1 = E + 1;  // <= kThreads
  int Ep = 1;
  while (Ep < E1) Ep <<= 1;
  const int P = kThreads / Ep;  // workgroup rows of H split in P parts per key
  const int e = tid % Ep, p = tid / Ep;
  const int r0 = (int)((int64_t)NB * p / P), r1 = (int)((int64_t)NB * (p + 1) / P);
  int sum = 0;
  if (e < E1)
    for (int r = r0; r < r1; ++r) sum += H[(int64_t)r * E1 + e];
  part[tid] = sum;
  __syncthreads();
  if (e < E1) {
    int run = 0, all = 0;
    for (int q = 0; q < P; ++q) {
      const int c = part[q * Ep + e];
      if (q < p) run += c;
      all += c;
    }
    if (p == 0) tot[e] = all;
    for (int r = r0; r < r1; ++r) {
      const int c = H[(int64_t)r * E1 + e];
      H[(int64_t)r * E1 + e] = run;
      run += c;
    }
  }
  __syncthreads();
  // as step B of the one-workgroup kernel
  const int g = tid;
  const int total = g < E ? tot[g] : 0;
  const int n_inv = tot[E];
  const int kept = g < E ? (total < cap ? total : cap) : 0;
  int n_over = 0, n_kept = 0;
  const int over_base = n_inv + block_exclusive_scan(g < E ? total - kept : 0, tmp, &n_over);
  const int kept_off = block_exclusive_scan(kept, tmp, &n_kept);
  const int n_drop = n_inv + n_over;
  const int Tk = (int)(T * k);
  if (g < E) {
    counts[g] = kept;
    offsets[g] = n_drop + kept_off;
    H[(int64_t)NB * E1 + g] = over_base;
  } else if (g < E + S) {
    counts[g] = (int)T;
    offsets[g] = Tk + (g - E) * (int)T;
  }
  if (g == 0) offsets[E + S] = Tk + S * (int)T;
}

__global__ __launch_bounds__(kThreads) void permute_place_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ slot_pos,
    const int32_t* __restrict__ H, const int32_t* __restrict__ offsets, int64_t n, int E,
    int NB, int cap) {
  __shared__ int32_t base[kThreads];      // [E + 1]: the key's copies in earlier workgroups
  __shared__ int32_t row_kept[kThreads];  // [E]
  __shared__ int32_t row_over[kThreads];  // [E]
  const int tid = threadIdx.x;
  const int E1 = E + 1;
  if (tid < E1) base[tid] = H[(int64_t)blockIdx.x * E1 + tid];
  if (tid < E) {
    row_kept[tid] = offsets[tid];
    row_over[tid] = H[(int64_t)NB * E1 + tid];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t s = (int64_t)blockIdx.x * kChunk + u * kThreads + tid;
    if (s >= n) continue;
    const int v = idx[s];
    const bool valid = v >= 0 && v < E;
    const int rank = base[valid ? v : E] + slot_pos[s];  // among the same key's copies
    const bool keep = valid && rank < cap;
    const int pos = !valid ? rank : keep ? row_kept[v] + rank : row_over[v] + rank - cap;
    slot_pos[s] = keep ? pos : -2 - pos;
  }
}

__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(
    int32_t* __restrict__ slot_pos, int32_t* __restrict__ sorted_slot, int64_t n) {
  const int64_t s = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (s >= n) return;
  const int v = slot_pos[s];
  sorted_slot[v >= 0 ? v : -2 - v] = (int32_t)s;
  if (v < 0) slot_pos[s] = -1;
}

}  // namespace

hipError_t launch_permute(const Shape& s, const int32_t* topk_idx, int64_t capacity,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                          int32_t* slot_pos, hipStream_t st) {
  int nbits = 0;
  while ((1 << nbits) <= s.E + 1) ++nbits;  // keys 0..E+1 (E: invalid id, E+1: idle lane)
  // no capacity, or one no expert can reach: every copy of a valid id is kept
  const int cap = capacity < 0 || capacity > s.Tk() ? (int)s.Tk() : (int)capacity;
  const int64_t n = s.Tk();
  const int64_t NB = (n + kChunk - 1) / kChunk;
  const int E1 = (int)s.E + 1;
  // the multi-workgroup form needs H ((NB + 1) x (E + 1)) to fit in
  // sorted_slot and at most kThreads keys
  if (n >= kMultiMin && E1 <= kThreads && (NB + 1) * E1 <= n) {
    int32_t* H = sorted_slot;
    const size_t lds = (size_t)kWaves * E1 * sizeof(int32_t);
    hipLaunchKernelGGL(permute_rank_kernel, dim3((unsigned)NB), dim3(kThreads), lds, st,
                       topk_idx, slot_pos, H, n, (int)s.E, nbits);
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kThreads), 0, st, H, counts, offsets,
                       s.T, s.k, (int)s.E, (int)s.S, (int)NB, cap);
    hipLaunchKernelGGL(permute_place_kernel, dim3((unsigned)NB), dim3(kThreads), 0, st,
                       topk_idx, slot_pos, (const int32_t*)H, (const int32_t*)offsets, n,
                       (int)s.E, (int)NB, cap);
    hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, st, slot_pos, sorted_slot, n);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kThreads), 0, st, topk_idx, counts,
                     offsets, sorted_slot, slot_pos, s.T, s.k, (int)s.E, (int)s.S,
                     nbits, cap);
  return hipGetLastError();
}

}  // namespace moe
