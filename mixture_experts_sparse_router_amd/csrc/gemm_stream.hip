// gemm_stream.hip -- grouped expert GEMM for decode-sized batches (groups of
// at most 64 rows), where the layer is bound by reading the active experts'
// weights from HBM once.
//
// Same operation and packed weight layout as the tiled kernels in gemm.hip
// (aitoday "MoEs in Transformers" page, sections "Dynamic Weight Loading with
// WeightConverter" and "Expert Backend"):
//   gate_up: act[r, n] = silu(x[t(r)] . Wgu[g, n]) * (x[t(r)] . Wgu[g, f+n])
//   down:    out[r, i] = act[r] . Wd[g, i]
//
// Each workgroup owns 16 output columns of one expert and streams those
// weight rows from HBM exactly once, straight into MFMA operand registers
// (4 waves split K); the few token rows ride along.  Kept in a file of its
// own so that it can be profiled and versioned apart from the prefill GEMM.
#include "decode_rows.h"

namespace moe {
namespace {

// One workgroup = 16 output columns of one expert group for all of the
// group's rows (16*MB rows per pass).  Its 4 waves split K: wave w takes the
// 128-wide K steps w, w+4, w+8, ..., so together they sweep each weight row
// front to back, and the 4 partial accumulators are added in LDS in wave
// order (fixed, so results are reproducible).  Lane (j = l%16, kb = l/16)
// loads, for chunk c of a K step, elements [k0 + 32c + 8kb, +8) of weight
// row n0+j and of token row j: 4 lanes cover 64 contiguous bytes of a row
// per load.
template <bool GATED, int MB, int CH, int NT>
struct StreamRegs {
  u32x4 bg[NT][CH], bu[NT][CH], a[MB][CH];
  bool ok[CH];  // chunk c lies inside K (else its registers are zeroed at use)
};

// Loads of one K step: the weight rows' chunks (of each of the NT column
// tiles) and the token rows' chunks.  Chunks past K read a valid address
// (offset 0) and are zeroed by a select when they are used, so the loads
// stay branch-free.
template <bool GATED, int MB, int CH, int NT>
__device__ __forceinline__ void stream_load_w(StreamRegs<GATED, MB, CH, NT>& r,
                                              const bf16_t* const* Bg, const bf16_t* const* Bu,
                                              int64_t k0, int kb, int64_t K) {
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t kk = k0 + 32 * c + 8 * kb;
    const bool ok = kk < K;
    const int64_t ka = ok ? kk : 0;
    r.ok[c] = ok;
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      r.bg[u][c] = ldg16(Bg[u] + ka);
      if constexpr (GATED) r.bu[u][c] = ldg16(Bu[u] + ka);
    }
  }
}
template <bool GATED, int MB, int CH, int NT>
__device__ __forceinline__ void stream_load_a(StreamRegs<GATED, MB, CH, NT>& r,
                                              const bf16_t* const* Ap, int64_t k0, int kb,
                                              int64_t K) {
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t kk = k0 + 32 * c + 8 * kb;
    const int64_t ka = kk < K ? kk : 0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) r.a[mb][c] = ldg16(Ap[mb] + ka);
  }
}

// FUSED (gate_up only): the group's rows are found from the expert ids
// themselves instead of a permutation (decode batches: at most 64 tokens),
// and the workgroups that hold column tile 0 write that permutation
// (counts, offsets, sorted_slot, slot_pos) for the steps that follow.
// PRE (gate_up only): out is float [R, 2N] and receives the pre-activation
// gate (column c) and up (column N + c) values instead of the SwiGLU (what
// the backward pass recomputes).
// NT column tiles of 16 per workgroup share each token-row load.
template <bool GATED, int MB, bool FUSED, int NW = 4, int U = 1, int CH = 4, bool PRE = false,
          int NT = 1>
__global__ __launch_bounds__(64 * NW) void stream_gemm_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ W,
    void* __restrict__ out_v, int64_t K, int64_t N, int64_t T, int64_t Tk, int64_t k,
    int G, int ntiles, const int32_t* __restrict__ topk_idx, int E,
    int32_t* __restrict__ p_counts, int32_t* __restrict__ p_offsets,
    int32_t* __restrict__ p_sorted, int32_t* __restrict__ p_slot_pos) {
  static_assert(GATED || !PRE, "pre-activation output of gate_up only");
  bf16_t* out = (bf16_t*)out_v;
  __shared__ f32x4 red[NW - 1][MB][NT][2][64];  // partials of waves 1..NW-1
  __shared__ int s_list[64];                    // FUSED: the group's copies, ascending
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ngroups = (ntiles + NT - 1) / NT;  // workgroups per expert group
  const int g = (int)blockIdx.x / ngroups;
  if (g >= G) return;
  const int tg = (int)blockIdx.x % ngroups;  // this workgroup's tiles: NT*tg ..
  const int j = lane & 15, kb = lane >> 4;
  int64_t col[NT];
  bool col_ok[NT];
  const bf16_t *Bg[NT], *Bu[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    col[u] = (int64_t)(tg * NT + u) * 16 + j;
    col_ok[u] = col[u] < N;
    const int64_t colc = col_ok[u] ? col[u] : N - 1;
    Bg[u] = W + ((int64_t)g * (GATED ? 2 * N : N) + colc) * K;
    Bu[u] = Bg[u] + N * K;  // up rows (GATED only)
  }
  // gate_up: the weights of this wave's first K step do not depend on the
  // group's rows, so their loads are issued before the group is looked up
  // (measured faster; an empty group drops them unused: at most one K step
  // per wave is read of an expert without rows)
  constexpr int KW = 32 * CH;  // K elements per step
  StreamRegs<GATED, MB, CH, NT> first;
  bool have_first = GATED;
  if constexpr (GATED)
    stream_load_w<GATED, MB, CH, NT>(first, Bg, Bu, (int64_t)wave * KW, kb, K);

  int64_t row_begin, rows;
  if constexpr (FUSED) {
    decode_group_rows(topk_idx, g, G, E, T, Tk, tg, wave, s_list,
                      DecodePerm{p_counts, p_offsets, p_sorted, p_slot_pos}, &row_begin, &rows);
  } else {
    row_begin = offsets[g];
    rows = offsets[g + 1] - row_begin;
  }
  if (rows <= 0) return;  // empty expert: its weights are never used

  for (int64_t m0 = 0; m0 < rows; m0 += 16 * MB) {
    const bf16_t* Ap[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      int64_t r = m0 + mb * 16 + j;
      if (r >= rows) r = rows - 1;  // padding rows repeat a valid row
      const int64_t grow = row_begin + r;
      if constexpr (FUSED) {
        Ap[mb] = A + decode_row_token(g, E, r, grow, Tk, T, k, s_list) * K;
      } else if constexpr (GATED) {
        Ap[mb] = A + row_token(grow, sorted_slot, Tk, k, T) * K;
      } else {
        Ap[mb] = A + grow * K;
      }
    }
    f32x4 accg[MB][NT], accu[MB][NT];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        accg[mb][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        accu[mb][u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    // U K steps per round (one by default: the other resident waves hide
    // the latency; more steps per round cost occupancy)
    for (int64_t k0 = (int64_t)wave * KW; k0 < K; k0 += (int64_t)KW * NW * U) {
      // U steps (k0, k0 + KW*NW, ...) loaded before any is used
      StreamRegs<GATED, MB, CH, NT> r[U];
#pragma unroll
      for (int v = 0; v < U; ++v) {
        const int64_t ku = k0 + (int64_t)KW * NW * v;
        if constexpr (GATED) {
          if (v == 0 && have_first) {
            r[0] = first;
            have_first = false;
          } else {
            stream_load_w<GATED, MB, CH, NT>(r[v], Bg, Bu, ku, kb, K);
          }
        } else {
          stream_load_w<GATED, MB, CH, NT>(r[v], Bg, Bu, ku, kb, K);
        }
        stream_load_a<GATED, MB, CH, NT>(r[v], Ap, ku, kb, K);
      }
#pragma unroll
      for (int v = 0; v < U; ++v) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
#pragma unroll
          for (int u = 0; u < NT; ++u) {
            const u32x4 bg = zero_unless(r[v].ok[c], r[v].bg[u][c]);
            const u32x4 bu = GATED ? zero_unless(r[v].ok[c], r[v].bu[u][c]) : bg;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              const u32x4 a = zero_unless(r[v].ok[c], r[v].a[mb][c]);
              accg[mb][u] = mfma16(a, bg, accg[mb][u]);
              if constexpr (GATED) accu[mb][u] = mfma16(a, bu, accu[mb][u]);
            }
          }
        }
      }
    }
    // add the NW K-split partials in wave order
    if (wave > 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          red[wave - 1][mb][u][0][lane] = accg[mb][u];
          if constexpr (GATED) red[wave - 1][mb][u][1][lane] = accu[mb][u];
        }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < NW - 1; ++w)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int u = 0; u < NT; ++u) {
            accg[mb][u] += red[w][mb][u][0][lane];
            if constexpr (GATED) accu[mb][u] += red[w][mb][u][1][lane];
          }
      // lane holds D[4*kb + q][j], q = 0..3, of each tile
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        if (!col_ok[u]) continue;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t r = m0 + mb * 16 + kb * 4 + q;
            if (r < rows) {
              if constexpr (PRE) {
                float* hrow = (float*)out_v + (row_begin + r) * 2 * N;
                hrow[col[u]] = accg[mb][u][q];
                hrow[N + col[u]] = accu[mb][u][q];
              } else {
                const float v = GATED ? swiglu(accg[mb][u][q], accu[mb][u][q]) : accg[mb][u][q];
                out[(row_begin + r) * N + col[u]] = f32_to_bf16(v);
              }
            }
          }
        }
      }
    }
    __syncthreads();  // red is reused by the next row pass
  }
}

}  // namespace

hipError_t launch_stream_gemm(bool gated, const Shape& s, const void* A,
                              const int32_t* sorted_slot, const int32_t* offsets, const void* W,
                              void* out, int64_t K, int64_t N, hipStream_t st) {
  const int G = (int)s.G();
  const int ntiles = (int)((N + 15) / 16);
  const unsigned grid = (unsigned)((int64_t)G * ntiles);
  const int MB = (int)((s.T + 15) / 16);
#define MOE_STREAM(gt, mb)                                                              \
  hipLaunchKernelGGL((stream_gemm_kernel<gt, mb, false>), dim3(grid), dim3(256), 0, st, \
                     (const bf16_t*)A, sorted_slot, offsets, (const bf16_t*)W,          \
                     (bf16_t*)out, K, N, s.T, s.Tk(), s.k, G, ntiles, nullptr, (int)s.E, \
                     nullptr, nullptr, nullptr, nullptr)
  if (gated) {
    switch (MB) {
      case 1:
        // two K steps loaded per round (measured 172 -> 166 us on the decode
        // gate_up; the fused form, which starts from its prefetched first
        // step, gains nothing from it and keeps one step per round)
        hipLaunchKernelGGL((stream_gemm_kernel<true, 1, false, 4, 2>), dim3(grid), dim3(256), 0,
                           st, (const bf16_t*)A, sorted_slot, offsets, (const bf16_t*)W,
                           (bf16_t*)out, K, N, s.T, s.Tk(), s.k, G, ntiles, nullptr, (int)s.E,
                           nullptr, nullptr, nullptr, nullptr);
        break;
      case 2: MOE_STREAM(true, 2); break;
      case 3: MOE_STREAM(true, 3); break;
      default: MOE_STREAM(true, 4); break;
    }
  } else {
    switch (MB) {
      case 1:
        // 8 waves (measured 85 -> 83 us on the decode down GEMM)
        hipLaunchKernelGGL((stream_gemm_kernel<false, 1, false, 8, 1>), dim3(grid), dim3(512), 0,
                           st, (const bf16_t*)A, sorted_slot, offsets, (const bf16_t*)W,
                           (bf16_t*)out, K, N, s.T, s.Tk(), s.k, G, ntiles, nullptr, (int)s.E,
                           nullptr, nullptr, nullptr, nullptr);
        break;
      case 2: MOE_STREAM(false, 2); break;
      case 3: MOE_STREAM(false, 3); break;
      default: MOE_STREAM(false, 4); break;
    }
  }
#undef MOE_STREAM
  return hipGetLastError();
}

hipError_t launch_stream_gate_up_preact(const Shape& s, const void* x, const int32_t* sorted_slot,
                                        const int32_t* offsets, const void* W_gate_up, float* H,
                                        hipStream_t st) {
  const int G = (int)s.G();
  const int ntiles = (int)((s.f + 15) / 16);
  const unsigned grid = (unsigned)((int64_t)G * ntiles);
  const int MB = (int)((s.T + 15) / 16);
#define MOE_PRE(mb)                                                                        \
  hipLaunchKernelGGL((stream_gemm_kernel<true, mb, false, 4, 1, 4, true>), dim3(grid),      \
                     dim3(256), 0, st, (const bf16_t*)x, sorted_slot, offsets,              \
                     (const bf16_t*)W_gate_up, H, s.d, s.f, s.T, s.Tk(), s.k, G, ntiles,     \
                     nullptr, (int)s.E, nullptr, nullptr, nullptr, nullptr)
  switch (MB) {
    case 1: MOE_PRE(1); break;
    case 2: MOE_PRE(2); break;
    case 3: MOE_PRE(3); break;
    default: MOE_PRE(4); break;
  }
#undef MOE_PRE
  return hipGetLastError();
}

hipError_t launch_gate_up_from_ids(const Shape& s, const void* x, const int32_t* topk_idx,
                                   const void* W_gate_up, void* act, int32_t* counts,
                                   int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos,
                                   hipStream_t st) {
  const int G = (int)s.G();
  const int ntiles = (int)((s.f + 15) / 16);
  const unsigned grid = (unsigned)((int64_t)G * ntiles);
  const int MB = (int)((s.T + 15) / 16);
#define MOE_FUSED(mb)                                                                   \
  hipLaunchKernelGGL((stream_gemm_kernel<true, mb, true>), dim3(grid), dim3(256), 0, st, \
                     (const bf16_t*)x, nullptr, nullptr, (const bf16_t*)W_gate_up,       \
                     (bf16_t*)act, s.d, s.f, s.T, s.Tk(), s.k, G, ntiles, topk_idx,      \
                     (int)s.E, counts, offsets, sorted_slot, slot_pos)
  switch (MB) {
    case 1: MOE_FUSED(1); break;
    case 2: MOE_FUSED(2); break;
    case 3: MOE_FUSED(3); break;
    default: MOE_FUSED(4); break;
  }
#undef MOE_FUSED
  return hipGetLastError();
}

}  // namespace moe
