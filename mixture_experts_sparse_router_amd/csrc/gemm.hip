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
#include <type_traits>

#include "moe_common.h"

namespace moe {
namespace {

// --------------------------------------------------------------- helpers


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
// Block tile BM x 256 (weight rows), 4 waves in a 2 x 2 grid, each
// wave BM/2 x 128 with v_mfma_f32_32x32x16_bf16 (the 16x16x32 form runs at
// half the rate on gfx950).  GATED: the 256 weight rows of a tile are 128
// gate rows and the 128 matching up rows, so wave column wn owns 64 output
// columns as 2 gate + 2 up 32-column blocks and SwiGLU pairs block ni with
// ni + 2 in registers.
//
// LDS: a ring of NST stages of A [BM][32] and B [256][32] bf16 (K tiles of
// 32), 64-byte rows whose 16-byte chunks are XOR-swizzled (swz below) so the
// 16-byte MFMA operand reads are bank-conflict free.  K tiles are copied
// global -> LDS directly (no registers) NST-1 tiles ahead; while the MFMAs
// of tile j run, tile j+1's operand fragments are read into a second
// register set.  One barrier per K tile.  Chunks past the end of K are
// copied from a 16-byte zero block.
//
// Tiles: m-tiles of every expert group (ceil(n_g / BM) each) times the
// n-tiles.  The host launches an upper bound; each workgroup computes the
// actual tile count from offsets and maps its id to a tile.  Workgroups are
// dealt to the 8 XCDs round robin, so ids with the same residue mod 8 get a
// contiguous run of the tile order, in which one expert group's tiles come
// as rectangles of its m-tiles by kBandN n-tiles.
constexpr int TBN = 256;        // weight rows per block tile

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// K per LDS stage and number of stages in the ring.
constexpr int SBK = 32;
constexpr int NST = 4;

// Element offset of logical 16-byte chunk c (0..3) of LDS row r (SBK bf16,
// 64 bytes per row).  The chunk is XOR-ed with (r >> 2) & 3, so the 16-byte
// operand reads of 16 consecutive rows at one logical chunk touch 16
// distinct 16-byte bank groups (the LDS serves 256 bytes per cycle).
__device__ __forceinline__ int swz(int r, int c) {
  return r * SBK + ((c ^ ((r >> 2) & 3)) << 3);
}

// n-tiles per band of the tile order: consecutive tiles of one expert group
// form (m-tiles x kBandN) rectangles, so workgroups running side by side on
// one XCD share both their activation rows and their weight panels in L2.
constexpr int kBandN = 4;

// Tile lookup: returns false for workgroups past the last tile.
__device__ bool find_tile(const int32_t* offsets, int G, int BM, int ntN, int bid, int* g_out,
                          int* mt_out, int* nt_out) {
  __shared__ int s_res[3];
  __shared__ int s_wave[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int c[4];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = tid * 4 + i;
    c[i] = g < G ? (offsets[g + 1] - offsets[g] + BM - 1) / BM : 0;  // m-tiles of g
    mine += c[i];
  }
  int inc = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) s_wave[wave] = inc;
  if (tid == 0) s_res[0] = -1;
  __syncthreads();
  const int total = (s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3]) * ntN;
  const int per = (total + 7) / 8;
  const int slot = bid >> 3;
  const int L = (bid & 7) * per + slot;  // XCD (bid mod 8) takes a contiguous run
  const bool valid = slot < per && L < total;
  int start = inc - mine;
  for (int w = 0; w < wave; ++w) start += s_wave[w];
  start *= ntN;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = c[i] * ntN;  // tiles of group tid*4+i
    if (valid && L >= start && L < start + n) {
      const int q = L - start;
      const int band = q / (c[i] * kBandN);
      const int bw = min(kBandN, ntN - band * kBandN);
      const int rem = q - band * c[i] * kBandN;
      s_res[0] = tid * 4 + i;
      s_res[1] = rem / bw;
      s_res[2] = band * kBandN + rem % bw;
    }
    start += n;
  }
  __syncthreads();
  *g_out = s_res[0];
  *mt_out = s_res[1];
  *nt_out = s_res[2];
  return s_res[0] >= 0;
}

// 16 zero bytes: the source of LDS chunks that lie past the end of K.
__device__ __attribute__((aligned(16))) bf16_t g_zero_chunk[8];

// Direct global -> LDS copy of 16 bytes per lane: lane l of the wave writes
// lds_base + 16*l.  No registers are involved, so the loads of the next K
// tile stay in flight for the whole of the current tile's MFMAs.
__device__ __forceinline__ void dma16(const void* src, bf16_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16,
                                   0, 0);
}

// One K tile of the tiled GEMM (see tiled_gemm_kernel).  The LDS slot being
// filled and the slot being read are separate __restrict__ parameters: once
// inlined, the compiler knows that the copies in flight never alias the
// operand reads and does not make the reads wait for them.
template <int MI, int NI, int AI, int BI, int ROWS_A>
__device__ __forceinline__ void gemm_tile_step(
    bf16_t* __restrict__ fillA, bf16_t* __restrict__ fillB, const bf16_t* __restrict__ readA,
    const bf16_t* __restrict__ readB, const bf16_t* const (&asrc)[AI], const int (&achunk)[AI],
    const bf16_t* const (&bsrc)[BI], const int (&bchunk)[BI], int64_t k0, int64_t K,
    const int (&arow)[MI], const int (&brow)[NI], int lh, int wave,
    const u32x4 (&cur)[2][MI + NI], u32x4 (&nxt)[2][MI + NI], f32x16 (&acc)[MI][NI]) {
  constexpr int NF = MI + NI;
  // tile j+1 has landed: this wave's copies, then everyone's (a plain
  // s_barrier: __syncthreads()'s release fence would wait for all copies)
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(1 * (AI + BI)) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // copy tile j+3 into the slot tile j-1 used
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int64_t kk = k0 + achunk[i];
    dma16(kk < K ? (const void*)(asrc[i] + kk) : (const void*)g_zero_chunk,
          fillA + (wave * (ROWS_A / 4) + 16 * i) * SBK);
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int64_t kk = k0 + bchunk[i];
    dma16(kk < K ? (const void*)(bsrc[i] + kk) : (const void*)g_zero_chunk,
          fillB + (wave * (TBN / 4) + 16 * i) * SBK);
  }
  // tile j+1's operand fragments
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      nxt[s][mi] = *reinterpret_cast<const u32x4*>(readA + swz(arow[mi], 2 * s + lh));
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      nxt[s][MI + ni] = *reinterpret_cast<const u32x4*>(readB + swz(brow[ni], 2 * s + lh));
  }
  // tile j's MFMAs
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = mfma32(cur[s][mi], cur[s][MI + ni], acc[mi][ni]);
  // order: copies, then the 2*NF LDS reads spread between the 2*MI*NI MFMAs
  __builtin_amdgcn_sched_group_barrier(0x020, AI + BI, 0);
#pragma unroll
  for (int i = 0; i < 2 * NF; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, MI * NI / NF, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * MI * NI - 2 * NF * (MI * NI / NF), 0);
}

template <bool GATED, int BM>
__global__ __launch_bounds__(256, 1) void tiled_gemm_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ W,
    bf16_t* __restrict__ out, int64_t K, int64_t N, int64_t T, int64_t Tk, int64_t k,
    int G, int ntN) {
  constexpr int MI = BM / 64;         // 32-row blocks per wave
  constexpr int NI = 4;               // 32-column blocks per wave
  constexpr int AI = BM / 64;         // A copies (16 rows, 1 KB) per wave per stage
  constexpr int BI = TBN / 64;        // B copies per wave per stage
  constexpr int NF = MI + NI;         // operand fragments per K sub-step of 16
  // one LDS object per ring slot: the compiler can then see that copies into
  // one slot never alias reads of another and need not wait for them
  __shared__ __attribute__((aligned(1024))) bf16_t sA0[BM * SBK], sA1[BM * SBK],
      sA2[BM * SBK], sA3[BM * SBK];
  __shared__ __attribute__((aligned(1024))) bf16_t sB0[TBN * SBK], sB1[TBN * SBK],
      sB2[TBN * SBK], sB3[TBN * SBK];
  static_assert(NST == 4, "four ring slots");
  static_assert(NST - 3 == 1, "gemm_tile_step waits for NST-3 = 1 later tile");
  auto slotA = [&](auto st) -> bf16_t* {
    if constexpr (decltype(st)::value == 0) return sA0;
    else if constexpr (decltype(st)::value == 1) return sA1;
    else if constexpr (decltype(st)::value == 2) return sA2;
    else return sA3;
  };
  auto slotB = [&](auto st) -> bf16_t* {
    if constexpr (decltype(st)::value == 0) return sB0;
    else if constexpr (decltype(st)::value == 1) return sB1;
    else if constexpr (decltype(st)::value == 2) return sB2;
    else return sB3;
  };
  int g, mt, nt;
  if (!find_tile(offsets, G, BM, ntN, (int)blockIdx.x, &g, &mt, &nt)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t row_begin = offsets[g] + (int64_t)mt * BM;
  const int64_t rows_left = offsets[g + 1] - row_begin;
  const int rows = (int)(rows_left < BM ? rows_left : BM);
  const int64_t ncols = GATED ? TBN / 2 : TBN;
  const int64_t n0 = (int64_t)nt * ncols;

  // ---- copy plan: wave w fills A rows [w*BM/4, (w+1)*BM/4) and B rows
  // [64w, 64w+64), 16 rows (1 KB) per copy.  Lane l lands on row l/4,
  // physical chunk l%4, which holds logical chunk (l%4) ^ ((row >> 2) & 3).
  const int lrow = lane >> 2;
  const int lphys = lane & 3;
  const bf16_t* asrc[AI];
  int achunk[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = wave * (BM / 4) + 16 * i + lrow;
    const int rc = r < rows ? r : rows - 1;  // padding rows repeat a valid row
    const int64_t grow = row_begin + rc;
    if constexpr (GATED) {
      asrc[i] = A + row_token(grow, sorted_slot, Tk, k, T) * K;
    } else {
      asrc[i] = A + grow * K;
    }
    achunk[i] = (lphys ^ ((r >> 2) & 3)) * 8;
  }
  const bf16_t* bsrc[BI];
  int bchunk[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int br = wave * (TBN / 4) + 16 * i + lrow;  // 0..255
    int64_t wrow;
    if constexpr (GATED) {
      int64_t c = n0 + (br & 127);
      if (c >= N) c = N - 1;
      wrow = (int64_t)g * 2 * N + (br < 128 ? c : N + c);
    } else {
      int64_t c = n0 + br;
      if (c >= N) c = N - 1;
      wrow = (int64_t)g * N + c;
    }
    bsrc[i] = W + wrow * K;
    bchunk[i] = (lphys ^ ((br >> 2) & 3)) * 8;
  }
  const int nk = (int)((K + SBK - 1) / SBK);
  // copy K tile j (clamped to the last tile) into ring slot st = j % NST
  auto issue = [&](auto st, int j) {
    j = j < nk ? j : nk - 1;
    const int64_t k0 = (int64_t)j * SBK;
    bf16_t* a = slotA(st);
    bf16_t* b = slotB(st);
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int64_t kk = k0 + achunk[i];
      dma16(kk < K ? (const void*)(asrc[i] + kk) : (const void*)g_zero_chunk,
            a + (wave * (BM / 4) + 16 * i) * SBK);
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int64_t kk = k0 + bchunk[i];
      dma16(kk < K ? (const void*)(bsrc[i] + kk) : (const void*)g_zero_chunk,
            b + (wave * (TBN / 4) + 16 * i) * SBK);
    }
  };

  // ---- wave sub-tile
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;
  int arow[MI], brow[NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) arow[mi] = wm * (BM / 2) + mi * 32 + lr;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    if constexpr (GATED) {
      // ni 0,1: gate columns 64wn + 32ni; ni 2,3: the matching up columns
      brow[ni] = (ni < 2 ? 0 : 128) + 64 * wn + 32 * (ni & 1) + lr;
    } else {
      brow[ni] = 128 * wn + 32 * ni + lr;
    }
  }
  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.f;

  // operand fragments of the K tile in ring slot st (2 sub-steps of 16)
  auto frags = [&](auto st, u32x4 (&f)[2][NF]) {
    const bf16_t* a = slotA(st);
    const bf16_t* b = slotB(st);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        f[s][mi] = *reinterpret_cast<const u32x4*>(a + swz(arow[mi], 2 * s + lh));
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        f[s][MI + ni] = *reinterpret_cast<const u32x4*>(b + swz(brow[ni], 2 * s + lh));
    }
  };
  // One K tile j in ring slot st: see gemm_tile_step.
  auto step = [&](auto st, int j, u32x4 (&cur)[2][NF], u32x4 (&nxt)[2][NF]) {
    constexpr int S = decltype(st)::value;
    using Fill = std::integral_constant<int, (S + NST - 1) % NST>;
    using Read = std::integral_constant<int, (S + 1) % NST>;
    const int jf = j + NST - 1 < nk ? j + NST - 1 : nk - 1;  // clamped copy
    gemm_tile_step<MI, NI, AI, BI, BM>(slotA(Fill{}), slotB(Fill{}), slotA(Read{}),
                                       slotB(Read{}), asrc, achunk, bsrc, bchunk,
                                       (int64_t)jf * SBK, K, arow, brow, lh, wave, cur, nxt,
                                       acc);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  u32x4 f0[2][NF], f1[2][NF];
  issue(S0{}, 0);
  issue(S1{}, 1);
  issue(S2{}, 2);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NST - 2) * (AI + BI)) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  frags(S0{}, f0);
  int kt = 0;
  for (; kt + 4 <= nk; kt += 4) {
    step(S0{}, kt, f0, f1);
    step(S1{}, kt + 1, f1, f0);
    step(S2{}, kt + 2, f0, f1);
    step(S3{}, kt + 3, f1, f0);
  }
  if (kt < nk) step(S0{}, kt, f0, f1);
  if (kt + 1 < nk) step(S1{}, kt + 1, f1, f0);
  if (kt + 2 < nk) step(S2{}, kt + 2, f0, f1);
  // drain the copies still in flight before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: lane holds D[8*(q/4) + 4*lh + (q%4)][lr] of each 32x32 block
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = wm * (BM / 2) + mi * 32 + 8 * (q >> 2) + 4 * lh + (q & 3);
      if (r >= rows) continue;
      bf16_t* orow = out + (row_begin + r) * N;
      if constexpr (GATED) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int64_t c = n0 + 64 * wn + 32 * ni + lr;
          if (c < N) orow[c] = f32_to_bf16(swiglu(acc[mi][ni][q], acc[mi][ni + 2][q]));
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int64_t c = n0 + 128 * wn + 32 * ni + lr;
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
  // rows per m-tile: 256 when groups are large on average, else 128
  const int64_t avg_rows = s.R() / (s.G() > 0 ? s.G() : 1);
  const int64_t ncols = GATED ? TBN / 2 : TBN;
  const int ntN = (int)((N + ncols - 1) / ncols);
  if (avg_rows >= 192) {
    const unsigned grid = ((mtile_bound(s, 256) * (unsigned)ntN) + 7u) & ~7u;
    hipLaunchKernelGGL((tiled_gemm_kernel<GATED, 256>), dim3(grid), dim3(256), 0, st,
                       (const bf16_t*)A, sorted_slot, offsets, (const bf16_t*)W, (bf16_t*)out,
                       K, N, s.T, s.Tk(), s.k, G, ntN);
  } else {
    const unsigned grid = ((mtile_bound(s, 128) * (unsigned)ntN) + 7u) & ~7u;
    hipLaunchKernelGGL((tiled_gemm_kernel<GATED, 128>), dim3(grid), dim3(256), 0, st,
                       (const bf16_t*)A, sorted_slot, offsets, (const bf16_t*)W, (bf16_t*)out,
                       K, N, s.T, s.Tk(), s.k, G, ntN);
  }
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
