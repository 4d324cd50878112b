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
#include "moe_common.h"

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
template <bool GATED, int MB>
struct StreamRegs {
  u32x4 bg[4], bu[4], a[MB][4];
  bool ok[4];  // chunk c lies inside K (else its registers are zeroed at use)
};

// Loads of one K step.  Chunks past K read a valid address (offset 0) and
// are zeroed by a select when they are used, so the loads stay branch-free.
template <bool GATED, int MB>
__device__ __forceinline__ void stream_load(StreamRegs<GATED, MB>& r, const bf16_t* Bg,
                                            const bf16_t* Bu, const bf16_t* const* Ap,
                                            int64_t k0, int kb, int64_t K) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t kk = k0 + 32 * c + 8 * kb;
    const bool ok = kk < K;
    const int64_t ka = ok ? kk : 0;
    r.ok[c] = ok;
    r.bg[c] = ldg16(Bg + ka);
    if constexpr (GATED) r.bu[c] = ldg16(Bu + ka);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) r.a[mb][c] = ldg16(Ap[mb] + ka);
  }
}

template <bool GATED, int MB>
__global__ __launch_bounds__(256) void stream_gemm_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ W,
    bf16_t* __restrict__ out, int64_t K, int64_t N, int64_t T, int64_t Tk, int64_t k,
    int G, int ntiles) {
  __shared__ f32x4 red[3][MB][2][64];  // partials of waves 1..3
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = (int)blockIdx.x / ntiles;
  if (g >= G) return;
  const int64_t row_begin = offsets[g];
  const int64_t rows = offsets[g + 1] - row_begin;
  if (rows <= 0) return;  // empty expert: its weights are never read
  const int j = lane & 15, kb = lane >> 4;
  const int64_t n0 = (int64_t)((int)blockIdx.x % ntiles) * 16;
  const int64_t col = n0 + j;
  const bool col_ok = col < N;
  const int64_t colc = col_ok ? col : N - 1;
  const bf16_t* Bg = W + ((int64_t)g * (GATED ? 2 * N : N) + colc) * K;
  const bf16_t* Bu = Bg + N * K;  // up rows (GATED only)

  for (int64_t m0 = 0; m0 < rows; m0 += 16 * MB) {
    const bf16_t* Ap[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      int64_t r = m0 + mb * 16 + j;
      if (r >= rows) r = rows - 1;  // padding rows repeat a valid row
      const int64_t grow = row_begin + r;
      if constexpr (GATED) {
        Ap[mb] = A + row_token(grow, sorted_slot, Tk, k, T) * K;
      } else {
        Ap[mb] = A + grow * K;
      }
    }
    f32x4 accg[MB], accu[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      accg[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      accu[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // one K step at a time: latency is hidden by the other resident waves
    // (explicit two-step register pipelining measured slower: it lowers
    // occupancy more than it adds bytes in flight)
    for (int64_t k0 = (int64_t)wave * 128; k0 < K; k0 += 512) {
      StreamRegs<GATED, MB> r;
      stream_load<GATED, MB>(r, Bg, Bu, Ap, k0, kb, K);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 bg = zero_unless(r.ok[c], r.bg[c]);
        const u32x4 bu = GATED ? zero_unless(r.ok[c], r.bu[c]) : bg;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const u32x4 a = zero_unless(r.ok[c], r.a[mb][c]);
          accg[mb] = mfma16(a, bg, accg[mb]);
          if constexpr (GATED) accu[mb] = mfma16(a, bu, accu[mb]);
        }
      }
    }
    // add the four K-split partials in wave order
    if (wave > 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        red[wave - 1][mb][0][lane] = accg[mb];
        if constexpr (GATED) red[wave - 1][mb][1][lane] = accu[mb];
      }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < 3; ++w) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          accg[mb] += red[w][mb][0][lane];
          if constexpr (GATED) accu[mb] += red[w][mb][1][lane];
        }
      }
      // lane holds D[4*kb + q][j], q = 0..3
      if (col_ok) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t r = m0 + mb * 16 + kb * 4 + q;
            if (r < rows) {
              const float v = GATED ? swiglu(accg[mb][q], accu[mb][q]) : accg[mb][q];
              out[(row_begin + r) * N + col] = f32_to_bf16(v);
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
  hipLaunchKernelGGL((stream_gemm_kernel<gt, mb>), dim3(grid), dim3(256), 0, st,       \
                     (const bf16_t*)A, sorted_slot, offsets, (const bf16_t*)W,          \
                     (bf16_t*)out, K, N, s.T, s.Tk(), s.k, G, ntiles)
  if (gated) {
    switch (MB) {
      case 1: MOE_STREAM(true, 1); break;
      case 2: MOE_STREAM(true, 2); break;
      case 3: MOE_STREAM(true, 3); break;
      default: MOE_STREAM(true, 4); break;
    }
  } else {
    switch (MB) {
      case 1: MOE_STREAM(false, 1); break;
      case 2: MOE_STREAM(false, 2); break;
      case 3: MOE_STREAM(false, 3); break;
      default: MOE_STREAM(false, 4); break;
    }
  }
#undef MOE_STREAM
  return hipGetLastError();
}

}  // namespace moe
