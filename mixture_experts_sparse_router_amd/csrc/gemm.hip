// gemm.hip -- grouped expert GEMMs over the variable-size expert groups.
//
// Expert weights are packed, one tensor per projection, so that a single
// launch covers every expert (aitoday "MoEs in Transformers" page, section
// "Dynamic Weight Loading with WeightConverter": gate_up_proj stacks the
// experts on dim 0 and concatenates w1 then w3 on dim 1 -> [G, 2f, d];
// down_proj stacks them -> [G, d, f]).  Token copies arrive sorted by expert,
// so group g is the contiguous row range [offsets[g], offsets[g+1]) of the
// permuted buffers (same page, section "Expert Backend", grouped_mm).
//
//   gate_up: act[r, n] = silu(x[t(r)] . Wgu[g, n]) * (x[t(r)] . Wgu[g, f+n])
//   down:    out[r, i] = act[r] . Wd[g, i]
//
// Both operands are K-contiguous ("NT"), which is the native operand layout
// of the gfx950 MFMA: every lane loads 8 consecutive K elements (16 bytes).
// The gate and up rows of one output column are computed by the same lanes,
// so SwiGLU is applied to the fp32 accumulators before rounding to bf16.
//
// Kernels
//   stream_gemm  bf16, groups of at most 64 rows (decode-shaped).  Each
//                workgroup owns 16 output columns of one expert and streams
//                those weight rows from HBM exactly once, straight into MFMA
//                operand registers (4 waves split K); the few token rows ride
//                along.  HBM-bound.
//   tiled_gemm   bf16, large groups.  128x128 block tile, 4 waves of 64x64,
//                K staged through LDS in double-buffered 64-wide slices,
//                v_mfma_f32_16x16x32_bf16.  Tiles of empty groups are never
//                launched work; m-tiles are found on the device from offsets.
//   f32_gemm     fp32 inputs: LDS-tiled FMA (fp32 vector and matrix peaks are
//                equal on MI355X), 64x64 tiles.
#include "moe_common.h"

namespace moe {
namespace {

// --------------------------------------------------------------- helpers

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 zero_unless(bool ok, u32x4 v) {
  return u32x4{ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u};
}

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Block-cooperative lookup of m-tile `tile` in the device-side tile list:
// group g owns ceil(count_g / BM) consecutive m-tiles.  Returns false when the
// block index is past the last tile.  G <= 1024; blockDim.x == 256.
__device__ bool find_mtile(const int32_t* offsets, int G, int BM, int tile, int* g_out,
                           int* mt_out) {
  __shared__ int s_found[2];
  __shared__ int s_wave[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int c[4];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = tid * 4 + i;
    c[i] = g < G ? (offsets[g + 1] - offsets[g] + BM - 1) / BM : 0;
    mine += c[i];
  }
  int inc = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (tid == 0) s_found[0] = -1;
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  int start = base + inc - mine;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (tile >= start && tile < start + c[i]) {
      s_found[0] = tid * 4 + i;
      s_found[1] = tile - start;
    }
    start += c[i];
  }
  __syncthreads();
  *g_out = s_found[0];
  *mt_out = s_found[1];
  return s_found[0] >= 0;
}

// ============================================================ stream_gemm
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

// ============================================================= tiled_gemm
constexpr int TBM = 128;        // rows per block tile
constexpr int TBN = 128;        // weight rows per block tile (GATED: 64 gate + 64 up)
constexpr int TBK = 64;         // K per LDS stage
constexpr int TLD = TBK + 8;    // padded LDS row (144 bytes): conflict-free 16B reads

template <bool GATED>
__global__ __launch_bounds__(256) void tiled_gemm_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ W,
    bf16_t* __restrict__ out, int64_t K, int64_t N, int64_t T, int64_t Tk, int64_t k,
    int G) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][TBM * TLD];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][TBN * TLD];
  int g, mt;
  if (!find_mtile(offsets, G, TBM, (int)blockIdx.x, &g, &mt)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t row_begin = offsets[g] + (int64_t)mt * TBM;
  const int64_t rows_left = offsets[g + 1] - row_begin;
  const int64_t rows = rows_left < TBM ? rows_left : TBM;
  // output columns covered by this block
  const int64_t ncols = GATED ? TBN / 2 : TBN;
  const int64_t n0 = (int64_t)blockIdx.y * ncols;

  // ---- per-thread global source rows (4 A pieces + 4 B pieces of 16B)
  const int prow = tid >> 3;        // 0..31
  const int pcol = (tid & 7) * 8;   // element offset inside the 64-wide slice
  const bf16_t* asrc[4];
  const bf16_t* bsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t r = prow + 32 * i;
    if (r >= rows) r = rows - 1;
    const int64_t grow = row_begin + r;
    if constexpr (GATED) {
      asrc[i] = A + row_token(grow, sorted_slot, Tk, k, T) * K + pcol;
    } else {
      asrc[i] = A + grow * K + pcol;
    }
    const int br = prow + 32 * i;  // 0..127
    int64_t wrow;
    if constexpr (GATED) {
      int64_t c = n0 + (br & 63);
      if (c >= N) c = N - 1;
      wrow = (int64_t)g * 2 * N + (br < 64 ? c : N + c);
    } else {
      int64_t c = n0 + br;
      if (c >= N) c = N - 1;
      wrow = (int64_t)g * N + c;
    }
    bsrc[i] = W + wrow * K + pcol;
  }

  const u32x4 z{0u, 0u, 0u, 0u};
  u32x4 ra[4], rb[4];
  auto gload = [&](int64_t k0) {
    const bool ok = k0 + pcol < K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ok ? ldg16(asrc[i] + k0) : z;
      rb[i] = ok ? ldg16(bsrc[i] + k0) : z;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&sA[buf][(prow + 32 * i) * TLD + pcol]) = ra[i];
      *reinterpret_cast<u32x4*>(&sB[buf][(prow + 32 * i) * TLD + pcol]) = rb[i];
    }
  };

  // ---- wave sub-tile: rows wm*64 .. +64; weight rows per the GATED layout
  const int wm = wave >> 1, wn = wave & 1;
  const int j = lane & 15, kb = lane >> 4;
  int brow[4];  // LDS B rows of the 4 column blocks this wave multiplies
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    if constexpr (GATED) {
      // ni 0,1: gate columns 32wn + 16ni; ni 2,3: the matching up columns
      brow[ni] = (ni < 2 ? 0 : 64) + 32 * wn + 16 * (ni & 1) + j;
    } else {
      brow[ni] = 64 * wn + 16 * ni + j;
    }
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)((K + TBK - 1) / TBK);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((int64_t)(kt + 1) * TBK);
#pragma unroll
    for (int ks = 0; ks < TBK / 32; ++ks) {
      u32x4 af[4], bfr[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *reinterpret_cast<const u32x4*>(
            &sA[cur][(wm * 64 + mi * 16 + j) * TLD + ks * 32 + kb * 8]);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        bfr[ni] = *reinterpret_cast<const u32x4*>(
            &sB[cur][brow[ni] * TLD + ks * 32 + kb * 8]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma16(af[mi], bfr[ni], acc[mi][ni]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds D[4*kb + q][j] of each 16x16 block
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t r = wm * 64 + mi * 16 + kb * 4 + q;
      if (r >= rows) continue;
      bf16_t* orow = out + (row_begin + r) * N;
      if constexpr (GATED) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int64_t c = n0 + 32 * wn + 16 * ni + j;
          if (c < N) orow[c] = f32_to_bf16(swiglu(acc[mi][ni][q], acc[mi][ni + 2][q]));
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int64_t c = n0 + 64 * wn + 16 * ni + j;
          if (c < N) orow[c] = f32_to_bf16(acc[mi][ni][q]);
        }
      }
    }
  }
}

// ================================================================ f32_gemm
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <bool GATED>
__global__ __launch_bounds__(256) void f32_gemm_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ offsets, const float* __restrict__ W,
    float* __restrict__ out, int64_t K, int64_t N, int64_t T, int64_t Tk, int64_t k,
    int G) {
  __shared__ float sA[FBK][FBM + 4];
  __shared__ float sB[FBK][FBN + 4];
  int g, mt;
  if (!find_mtile(offsets, G, FBM, (int)blockIdx.x, &g, &mt)) return;
  const int tid = threadIdx.x;
  const int64_t row_begin = offsets[g] + (int64_t)mt * FBM;
  const int64_t rows_left = offsets[g + 1] - row_begin;
  const int64_t rows = rows_left < FBM ? rows_left : FBM;
  const int64_t ncols = GATED ? FBN / 2 : FBN;
  const int64_t n0 = (int64_t)blockIdx.y * ncols;

  // loader: thread -> (row lr = tid/4, k quad lk = (tid%4)*4) for A and B
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  int64_t ar = lr < rows ? lr : rows - 1;
  const int64_t agrow = row_begin + ar;
  const float* asrc =
      GATED ? A + row_token(agrow, sorted_slot, Tk, k, T) * K : A + agrow * K;
  int64_t wrow;
  if constexpr (GATED) {
    int64_t c = n0 + (lr & 31);
    if (c >= N) c = N - 1;
    wrow = (int64_t)g * 2 * N + (lr < 32 ? c : N + c);
  } else {
    int64_t c = n0 + lr;
    if (c >= N) c = N - 1;
    wrow = (int64_t)g * N + c;
  }
  const float* bsrc = W + wrow * K;

  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += FBK) {
    const int64_t kk = k0 + lk;
    float4 va = make_float4(0.f, 0.f, 0.f, 0.f), vb = va;
    if (kk < K) {  // K % 8 == 0, so a quad is all in or all out
      va = *reinterpret_cast<const float4*>(asrc + kk);
      vb = *reinterpret_cast<const float4*>(bsrc + kk);
    }
    sA[lk + 0][lr] = va.x; sA[lk + 1][lr] = va.y; sA[lk + 2][lr] = va.z; sA[lk + 3][lr] = va.w;
    sB[lk + 0][lr] = vb.x; sB[lk + 1][lr] = vb.y; sB[lk + 2][lr] = vb.z; sB[lk + 3][lr] = vb.w;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < FBK; ++q) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[q][ty * 4 + i];
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = sB[q][tx + 16 * i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c] = fmaf(a[i], b[c], acc[i][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = ty * 4 + i;
    if (r >= rows) continue;
    float* orow = out + (row_begin + r) * N;
    if constexpr (GATED) {
      // B columns tx, tx+16 are gate columns; tx+32, tx+48 the matching up ones
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int64_t col = n0 + tx + 16 * c;
        if (col < N) orow[col] = swiglu(acc[i][c], acc[i][c + 2]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int64_t col = n0 + tx + 16 * c;
        if (col < N) orow[col] = acc[i][c];
      }
    }
  }
}

// ---------------------------------------------------------------- launch

// Upper bound of the m-tiles of all groups: sum ceil(n_g/BM) <= R/BM + groups.
inline unsigned mtile_bound(const Shape& s, int BM) {
  const int64_t R = s.R();
  int64_t nonempty = s.G() < R ? s.G() : R;
  return (unsigned)(R / BM + nonempty + 1);
}

template <bool GATED>
hipError_t launch_bf16(const Shape& s, const void* A, const int32_t* sorted_slot,
                       const int32_t* offsets, const void* W, void* out, int64_t K,
                       int64_t N, hipStream_t st) {
  const int G = (int)s.G();
  if (s.T <= 64) {
    const int ntiles = (int)((N + 15) / 16);
    const unsigned grid = (unsigned)((int64_t)G * ntiles);
    const int MB = (int)((s.T + 15) / 16);
#define MOE_STREAM(mb)                                                                 \
  hipLaunchKernelGGL((stream_gemm_kernel<GATED, mb>), dim3(grid), dim3(256), 0, st,    \
                     (const bf16_t*)A, sorted_slot, offsets, (const bf16_t*)W,         \
                     (bf16_t*)out, K, N, s.T, s.Tk(), s.k, G, ntiles)
    switch (MB) {
      case 1: MOE_STREAM(1); break;
      case 2: MOE_STREAM(2); break;
      case 3: MOE_STREAM(3); break;
      default: MOE_STREAM(4); break;
    }
#undef MOE_STREAM
    return hipGetLastError();
  }
  const int64_t ncols = GATED ? TBN / 2 : TBN;
  dim3 grid(mtile_bound(s, TBM), (unsigned)((N + ncols - 1) / ncols));
  hipLaunchKernelGGL((tiled_gemm_kernel<GATED>), grid, dim3(256), 0, st, (const bf16_t*)A,
                     sorted_slot, offsets, (const bf16_t*)W, (bf16_t*)out, K, N, s.T,
                     s.Tk(), s.k, G);
  return hipGetLastError();
}

template <bool GATED>
hipError_t launch_f32(const Shape& s, const void* A, const int32_t* sorted_slot,
                      const int32_t* offsets, const void* W, void* out, int64_t K,
                      int64_t N, hipStream_t st) {
  const int64_t ncols = GATED ? FBN / 2 : FBN;
  dim3 grid(mtile_bound(s, FBM), (unsigned)((N + ncols - 1) / ncols));
  hipLaunchKernelGGL((f32_gemm_kernel<GATED>), grid, dim3(256), 0, st, (const float*)A,
                     sorted_slot, offsets, (const float*)W, (float*)out, K, N, s.T, s.Tk(),
                     s.k, (int)s.G());
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const Shape& s, const void* x, const int32_t* sorted_slot,
                          const int32_t* offsets, const void* W_gate_up, void* act,
                          hipStream_t st) {
  if (s.R() == 0) return hipSuccess;
  if (s.dt == MOE_DT_BF16)
    return launch_bf16<true>(s, x, sorted_slot, offsets, W_gate_up, act, s.d, s.f, st);
  return launch_f32<true>(s, x, sorted_slot, offsets, W_gate_up, act, s.d, s.f, st);
}

hipError_t launch_down(const Shape& s, const void* act, const int32_t* offsets,
                       const void* W_down, void* expert_out, hipStream_t st) {
  if (s.R() == 0) return hipSuccess;
  if (s.dt == MOE_DT_BF16)
    return launch_bf16<false>(s, act, nullptr, offsets, W_down, expert_out, s.f, s.d, st);
  return launch_f32<false>(s, act, nullptr, offsets, W_down, expert_out, s.f, s.d, st);
}

}  // namespace moe
