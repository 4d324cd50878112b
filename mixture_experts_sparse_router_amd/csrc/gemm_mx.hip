// gemm_mx.hip -- grouped expert GEMMs with MXFP4 expert weights, for
// decode-sized batches (at most 64 tokens), where the layer is bound by
// reading the active experts' weights.
//
// The aitoday "MoEs in Transformers" page (section "From Dense to Sparse")
// notes that generation would be faster still with kernels for the model's
// native mxfp4 quantisation, and (section "Dynamic Weight Loading with
// WeightConverter") that per-expert quantisation relies on the packed expert
// layout.  Format (OCP Microscaling, which the pages name but do not
// define): FP4 E2M1 elements, two per byte (even element in the low nibble),
// and one E8M0 scale byte X (factor 2^(X-127)) for each run of 32
// consecutive elements of a weight row.  Tensors keep the packed expert
// layout of the bf16 weights:
//   gate_up: Wq [G, 2f, d/2], Ws [G, 2f, d/32]   down: Wq [G, d, f/2], Ws [G, d, f/32]
// Weight-only: activations stay bf16, so the layer computes exactly what the
// bf16 layer computes on the dequantised weights (every dequantised value is
// a bf16 number: 2 significant bits times a power of two).
//
// Same work split as the bf16 decode kernel (gemm_stream.hip): one
// workgroup = 16 output columns (NT x 16 for the down GEMM of one row
// block) of one expert for all of its rows, 4 waves
// splitting K into 128-wide steps.  Lane (j = l%16, kb = l/16) loads, per K
// step, the 32-element block [k0 + 32kb, +32) of weight row n0 + j: 16
// contiguous bytes and its one scale byte (so 4 lanes cover 64 contiguous
// bytes of a row).  gfx950 converts FP4 to bf16 with the scale applied in
// one instruction per byte (v_cvt_scalef32_pk_bf16_fp4: byte -> two bf16,
// low nibble first, times 2^(X-127) taken from the exponent field of the
// fp32 scale operand); dword c of the block feeds 16x16x32 MFMA c, whose
// token operand is the same lane's elements [k0 + 32kb + 8c, +8).  U steps
// are loaded before any is used, to keep enough bytes in flight with a
// quarter of the bf16 kernel's weight bytes per step: for one block of 16
// rows, U is the smallest of 2, 4, 6 whose round covers K (measured: at
// K = 2880 one round of U = 6 beats two rounds of U = 4 by 20%, and U = 8
// lowers occupancy); more rows leave fewer registers for steps.
#include "decode_rows.h"

namespace moe {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Eight FP4 elements (one dword) times 2^(X-127) -> eight bf16 (one MFMA
// operand).  scale: fp32 whose exponent field is X.
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t w, float scale) {
  return u32x4{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3))};
}

template <bool GATED, int MB, int NT>
struct MxStep {
  u32x4 qg[NT], qu[NT];     // 32 packed FP4 elements of each tile's gate (and up) row
  uint32_t sg[NT], su[NT];  // their E8M0 scale bytes
  u32x4 a[MB][4];           // token rows' elements [k0 + 32kb + 8c, +8), c = 0..3
  bool ok;                  // the block lies inside K (else used as zeros)
};

// FUSED (gate_up only): the group's rows are found from the expert ids and
// the workgroups that hold column tile 0 write the permutation
// (decode_rows.h), so the layer needs no permutation launch.
// NT column tiles of 16 per workgroup: each token-row chunk a lane loads
// feeds NT weight tiles (the token rows are re-read from L2 by every
// workgroup of the group; with 4-bit weights they would otherwise be two
// thirds of the bytes a workgroup moves).
template <bool GATED, int MB, int U, int NW, bool FUSED = false, int NT = 1>
__global__ __launch_bounds__(64 * NW) void stream_mx_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ offsets, const uint8_t* __restrict__ Wq,
    const uint8_t* __restrict__ Ws, bf16_t* __restrict__ out, int64_t K, int64_t N,
    int64_t T, int64_t Tk, int64_t k, int G, int ntiles, const int32_t* __restrict__ topk_idx,
    int E, DecodePerm perm) {
  static_assert(GATED || !FUSED, "fused row lookup in gate_up only");
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
  const uint8_t *qg[NT], *qu[NT], *sgp[NT], *sup[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    col[u] = (int64_t)(tg * NT + u) * 16 + j;
    col_ok[u] = col[u] < N;
    const int64_t colc = col_ok[u] ? col[u] : N - 1;
    const int64_t wrow = (int64_t)g * (GATED ? 2 * N : N) + colc;  // gate (or down) row
    qg[u] = Wq + wrow * (K / 2);
    qu[u] = qg[u] + N * (K / 2);  // up row (GATED only)
    sgp[u] = Ws + wrow * (K / 32);
    sup[u] = sgp[u] + N * (K / 32);
  }
  int64_t row_begin, rows;
  if constexpr (FUSED) {
    decode_group_rows(topk_idx, g, G, E, T, Tk, tg, wave, s_list, perm, &row_begin, &rows);
  } else {
    row_begin = offsets[g];
    rows = offsets[g + 1] - row_begin;
  }
  if (rows <= 0) return;  // empty expert: its weights are never read

  for (int64_t m0 = 0; m0 < rows; m0 += 16 * MB) {
    const bf16_t* Ap[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      int64_t r = m0 + mb * 16 + j;
      if (r >= rows) r = rows - 1;  // padding rows repeat a valid row
      const int64_t grow = row_begin + r;
      if constexpr (FUSED)
        Ap[mb] = A + decode_row_token(g, E, r, grow, Tk, T, k, s_list) * K;
      else
        Ap[mb] = A + (GATED ? row_token(grow, sorted_slot, Tk, k, T) : grow) * K;
    }
    f32x4 accg[MB][NT], accu[MB][NT];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        accg[mb][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        accu[mb][u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    // wave w takes the K steps w, w+NW, ...; U of them per round
    for (int64_t k0 = (int64_t)wave * 128; k0 < K; k0 += 128 * NW * U) {
      MxStep<GATED, MB, NT> st[U];
#pragma unroll
      for (int v = 0; v < U; ++v) {
        const int64_t kk = k0 + 128 * NW * v + 32 * kb;  // the lane's 32-element block
        st[v].ok = kk < K;
        const int64_t ka = st[v].ok ? kk : 0;  // past K: block 0, zeroed at use
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          st[v].qg[u] = ldg16(qg[u] + ka / 2);
          st[v].sg[u] = sgp[u][ka / 32];
          if constexpr (GATED) {
            st[v].qu[u] = ldg16(qu[u] + ka / 2);
            st[v].su[u] = sup[u][ka / 32];
          }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int c = 0; c < 4; ++c) st[v].a[mb][c] = ldg16(Ap[mb] + ka + 8 * c);
      }
#pragma unroll
      for (int v = 0; v < U; ++v) {
        const bool ok = st[v].ok;
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          const float scg = __uint_as_float(st[v].sg[u] << 23);
          const float scu = __uint_as_float(st[v].su[u] << 23);
          const uint32_t wg[4] = {st[v].qg[u].x, st[v].qg[u].y, st[v].qg[u].z, st[v].qg[u].w};
          const uint32_t wu[4] = {st[v].qu[u].x, st[v].qu[u].y, st[v].qu[u].z, st[v].qu[u].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const u32x4 bg = zero_unless(ok, fp4x8_to_bf16(wg[c], scg));
            u32x4 bu = bg;
            if constexpr (GATED) bu = zero_unless(ok, fp4x8_to_bf16(wu[c], scu));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              const u32x4 a = zero_unless(ok, st[v].a[mb][c]);
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
              const float v = GATED ? swiglu(accg[mb][u][q], accu[mb][u][q]) : accg[mb][u][q];
              out[(row_begin + r) * N + col[u]] = f32_to_bf16(v);
            }
          }
        }
      }
    }
    __syncthreads();  // red is reused by the next row pass
  }
}

// The launch of one decode MXFP4 GEMM.  fused: gate_up with the rows found
// from topk_idx, writing the permutation into perm.
template <bool FUSED>
hipError_t launch_mx(bool gated, const Shape& s, const void* A, const int32_t* sorted_slot,
                     const int32_t* offsets, const uint8_t* Wq, const uint8_t* Ws, void* out,
                     int64_t K, int64_t N, const int32_t* topk_idx, const DecodePerm& perm,
                     hipStream_t st) {
  if (s.R() == 0) return hipSuccess;
  const int G = (int)s.G();
  const int ntiles = (int)((N + 15) / 16);
  const int MB = (int)((s.T + 15) / 16);
#define MOE_MX_NT(gt, mb, u, nt)                                                            \
  hipLaunchKernelGGL((stream_mx_kernel<gt, mb, u, 4, FUSED && gt, nt>),                     \
                     dim3((unsigned)((int64_t)G * ((ntiles + nt - 1) / nt))), dim3(256), 0,  \
                     st, (const bf16_t*)A, sorted_slot, offsets, Wq, Ws, (bf16_t*)out, K, N,   \
                     s.T, s.Tk(), s.k, G, ntiles, topk_idx, (int)s.E, perm)
#define MOE_MX(gt, mb, u) MOE_MX_NT(gt, mb, u, 1)
  const int u1 = K <= 1024 ? 2 : K <= 2048 ? 4 : 6;  // steps per round, one row block
  if (gated) {
    if (MB == 1) {
      if (u1 == 2) MOE_MX(true, 1, 2);
      else if (u1 == 4) MOE_MX(true, 1, 4);
      else MOE_MX(true, 1, 6);
    } else if (MB == 2) {
      MOE_MX(true, 2, 2);
    } else if (MB == 3) {
      MOE_MX(true, 3, 1);
    } else {
      MOE_MX(true, 4, 1);
    }
  } else {
    if (MB == 1) {
      // two column tiles per workgroup, two steps per round (measured at
      // d = f = 2880: 33.4 -> 28.2 us; the gate_up, with twice the weight
      // bytes per tile, is fastest with one tile and one round covering K)
      MOE_MX_NT(false, 1, 2, 2);
    } else if (MB == 2) {
      MOE_MX(false, 2, 2);
    } else if (MB == 3) {
      MOE_MX(false, 3, 1);
    } else {
      MOE_MX(false, 4, 1);
    }
  }
#undef MOE_MX
#undef MOE_MX_NT
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_mx(bool gated, const Shape& s, const void* A,
                            const int32_t* sorted_slot, const int32_t* offsets,
                            const uint8_t* Wq, const uint8_t* Ws, void* out, int64_t K,
                            int64_t N, hipStream_t st) {
  return launch_mx<false>(gated, s, A, sorted_slot, offsets, Wq, Ws, out, K, N, nullptr,
                          DecodePerm{}, st);
}

hipError_t launch_gate_up_mx_from_ids(const Shape& s, const void* x, const int32_t* topk_idx,
                                      const uint8_t* Wq, const uint8_t* Ws, void* act,
                                      int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                                      int32_t* slot_pos, hipStream_t st) {
  return launch_mx<true>(true, s, x, nullptr, nullptr, Wq, Ws, act, s.d, s.f, topk_idx,
                         DecodePerm{counts, offsets, sorted_slot, slot_pos}, st);
}

}  // namespace moe
