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
//   stream_gemm  bf16, T <= 64 (decode): in gemm_stream.hip.
//   tiled_gemm   bf16, larger batches.  BM x 256 block tile (BM = 128 or
//                256), 4 or 8 waves in a 2 x (2 or 4) grid,
//                v_mfma_f32_32x32x16_bf16; K tiles of 32 or 64 staged
//                through a ring of LDS stages by direct global -> LDS copies.
//                Tiles of empty groups are never launched work; m-tiles are
//                found on the device from offsets.
//   f32_gemm     fp32 inputs: LDS-tiled FMA (fp32 vector and matrix peaks are
//                equal on MI355X), 64x64 tiles.
#include <type_traits>
#include <utility>

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

// ============================================================= tiled_gemm
// Block tile BM x 256 (weight rows), NW = 4 or 8 waves in a 2 x NW/2 grid,
// each wave BM/2 x 512/NW with v_mfma_f32_32x32x16_bf16 (the 16x16x32 form
// runs at half the rate on gfx950).  GATED: the 256 weight rows of a tile
// are 128 gate rows and the 128 matching up rows, so wave column wn owns
// 256/NW output columns as gate blocks plus the matching up blocks, and
// SwiGLU pairs block ni with ni + NI/2 in registers.
//
// LDS: a ring of NST stages, each A [BM][SBK] and B [256][SBK] bf16 (K
// tiles of SBK = 32 or 64), rows of 64 or 128 bytes whose 16-byte chunks are
// XOR-swizzled so that the 16-byte MFMA operand reads are bank-conflict
// free.  K tiles are copied global -> LDS directly (buffer loads with the
// LDS bit, no registers) NST tiles ahead.  A K tile is SBK/16 MFMA
// sub-steps of K = 16; the operand fragments of the next sub-step are read
// from LDS into a second register set while the current sub-step's MFMAs
// run.  One barrier per K tile.
//
// Out-of-range elements come back as zeros from the buffer loads' range
// check: rows past the group (or past N), chunks past the end of K, and the
// whole of the copies issued for K tiles past the end, which keep the number
// of copies in flight the same on every step (and move no data).
//
// Tiles: m-tiles of every expert group (ceil(n_g / BM) each) times the
// n-tiles.  The host launches an upper bound; each workgroup computes the
// actual tile count from offsets and maps its id to a tile.  Workgroups are
// dealt to the 8 XCDs round robin, so ids with the same residue mod 8 get a
// contiguous run of the tile order, in which one expert group's tiles come
// as rectangles of its m-tiles by kBandN n-tiles.
constexpr int TBN = 256;  // weight rows per block tile
#ifndef MOE_PANEL_NST
#define MOE_PANEL_NST 4
#endif

// Scheduling of one MFMA sub-step: after MFMA I come items [I*N/NM,
// (I+1)*N/NM) of the sequence "NA items of kind KA, then NB of kind KB"
// (N = NA + NB, NM MFMAs), as sched_group_barrier groups.
template <int I, int NM, int NA, int KA, int NB, int KB>
__device__ __forceinline__ void sched_one() {
  constexpr int b = I * (NA + NB) / NM, e = (I + 1) * (NA + NB) / NM;
  constexpr int ba = b < NA ? b : NA, ea = e < NA ? e : NA;
  constexpr int na = ea - ba, nb = (e - b) - na;
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
  if constexpr (na > 0) __builtin_amdgcn_sched_group_barrier(KA, na, 0);
  if constexpr (nb > 0) __builtin_amdgcn_sched_group_barrier(KB, nb, 0);
}
template <int NM, int NA, int KA, int NB, int KB, int... Is>
__device__ __forceinline__ void sched_spread(std::integer_sequence<int, Is...>) {
  (sched_one<Is, NM, NA, KA, NB, KB>(), ...);
}
constexpr int kSchedVmem = 0x020, kSchedDsRead = 0x100;

// n-tiles per band of the tile order: consecutive tiles of one expert group
// form (m-tiles x kBandN) rectangles, so workgroups running side by side on
// one XCD share both their activation rows and their weight panels in L2.
constexpr int kBandN = 4;

// Tile lookup: returns false for workgroups past the last tile.
// NW waves per workgroup (4*64*NW >= 1024 groups covered); lds: 3 + NW
// ints of workgroup-shared scratch.
template <int NW>
__device__ bool find_tile(const int32_t* offsets, int G, int BM, int ntN, int bid, int* g_out,
                          int* mt_out, int* nt_out, int* lds) {
  int* s_res = lds;       // [3]
  int* s_wave = lds + 3;  // [NW]
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
  int total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) total += s_wave[w];
  total *= ntN;
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

// PRE (gate_up only): out is float [R, 2N] and receives the pre-activation
// gate (columns < N) and up (columns N + c) values instead of the SwiGLU
// (what the backward pass recomputes).
template <bool GATED, int BM, int NST, int OCC, int NW, int SBK, bool PRE = false>
__global__ __launch_bounds__(64 * NW, OCC) void tiled_gemm_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ W,
    void* __restrict__ out_v, int64_t K, int64_t N, int64_t T, int64_t Tk, int64_t k,
    int G, int ntN) {
  static_assert(GATED || !PRE, "pre-activation output of gate_up only");
  bf16_t* out = (bf16_t*)out_v;
  constexpr int WN = NW / 2;            // wave grid 2 x WN
  constexpr int MI = BM / 64;           // 32-row blocks per wave (BM/2 rows)
  constexpr int NI = 8 / WN;            // 32-column blocks per wave (256/WN columns)
  constexpr int CPR = SBK / 8;          // 16-byte chunks per LDS row (4 or 8)
  constexpr int RPC = 64 / CPR;         // rows per copy instruction (16 or 8)
  constexpr int NSUB = SBK / 16;        // MFMA sub-steps per K tile
  constexpr int AI = BM / (RPC * NW);   // A copies (1 KB each) per wave per stage
  constexpr int BI = TBN / (RPC * NW);  // B copies per wave per stage
  static_assert(SBK == 32 || SBK == 64, "K tile");
  static_assert(AI >= 1 && BI >= 1 && NI >= 2, "tile split");
  static_assert(BM % (RPC * NW) == 0 && TBN % (RPC * NW) == 0 && BM % 64 == 0, "copy plan");
  constexpr int NF = MI + NI;   // operand fragments per sub-step
  constexpr uint32_t ROWB = SBK * 2;         // bytes per LDS row
  constexpr uint32_t STA = BM * ROWB;         // bytes per stage of A
  constexpr uint32_t STB = TBN * ROWB;        // bytes per stage of B
  // two LDS objects (A and B stages): with more than one, the compiler tags
  // each LDS access with the object it touches
  __shared__ __attribute__((aligned(1024))) unsigned char ringA[NST * STA];
  __shared__ __attribute__((aligned(1024))) unsigned char ringB[NST * STB];

  static_assert(NST * (STA + STB) * OCC <= 160 * 1024, "ring fits the LDS");
  static_assert((NST - 1) * (AI + BI) < 64 && NST >= 2, "vmcnt range");

  int g, mt, nt;
  // the tile lookup's scratch lives at the start of the ring; the barrier
  // after it keeps the first copies from overwriting it while it is read
  if (!find_tile<NW>(offsets, G, BM, ntN, (int)blockIdx.x, &g, &mt, &nt,
                     reinterpret_cast<int*>(ringA)))
    return;
  __syncthreads();
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t row_begin = offsets[g] + (int64_t)mt * BM;
  const int64_t rows_left = offsets[g + 1] - row_begin;
  const int rows = (int)(rows_left < BM ? rows_left : BM);
  const int64_t ncols = GATED ? TBN / 2 : TBN;
  const int64_t n0 = (int64_t)nt * ncols;
  const uint32_t Kb = (uint32_t)(K * 2);  // bytes per operand row

  // ---- buffer resources.  A: gate_up gathers token rows from all of x;
  // down reads this tile's rows of act.  B: this expert's weight matrix.
  const bf16_t* abase = GATED ? A : A + row_begin * K;
  const uint32_t a_bytes = GATED ? (uint32_t)(T * K * 2) : (uint32_t)rows * Kb;
  const int64_t wrows = GATED ? 2 * N : N;
  const bf16_t* bbase = W + (int64_t)g * wrows * K;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)abase, 0, (int)a_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)bbase, 0, (int)(uint32_t)(wrows * K * 2),
                                        kRsrcWord3);

  // ---- copy plan: wave w fills A rows [w*BM/NW, (w+1)*BM/NW) and B rows
  // [w*256/NW, (w+1)*256/NW), RPC rows (1 KB) per copy.  Lane l lands on row
  // l/CPR of the copy, physical chunk l%CPR, which holds logical chunk
  // (l%CPR) ^ sw(row); sw(row) = (row / (16/CPR)) & (CPR-1) makes the 16-byte
  // reads of 16 consecutive rows hit 16 distinct bank groups.  For CPR = 4
  // the XOR term only depends on l; for CPR = 8 also on the copy's parity.
  const int lrow = lane / CPR;
  auto kchunk_of = [&](int first_row) {  // K element of the lane's chunk
    const int row = first_row + lrow;
    return ((lane % CPR) ^ ((row / (16 / CPR)) & (CPR - 1))) * 8;
  };
  uint32_t aoff[AI], boff[BI];  // byte offset of the lane's row + chunk, or kOOB
  int akc[AI], bkc[BI];         // the lane's K element within a tile
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r0 = wave * (BM / NW) + RPC * i;
    const int r = r0 + lrow;
    akc[i] = kchunk_of(r0);
    uint32_t o = kOOB;
    if (r < rows) {
      const int64_t src_row =
          GATED ? row_token(row_begin + r, sorted_slot, Tk, k, T) : (int64_t)r;
      o = (uint32_t)src_row * Kb + (uint32_t)akc[i] * 2;
    }
    aoff[i] = o;
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int b0 = wave * (TBN / NW) + RPC * i;
    const int br = b0 + lrow;  // 0..255
    bkc[i] = kchunk_of(b0);
    const int64_t c = n0 + (GATED ? (br & 127) : br);
    uint32_t o = kOOB;
    if (c < N) {
      const int64_t wrow = GATED ? (br < 128 ? c : N + c) : c;
      o = (uint32_t)wrow * Kb + (uint32_t)bkc[i] * 2;
    }
    boff[i] = o;
  }
  // the ring's LDS address as an integer for the copies, kept apart from the
  // pointer arithmetic of the fragment reads
  uint32_t ring_a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ringA;
  uint32_t ring_b = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ringB;
  asm("" : "+s"(ring_a), "+s"(ring_b));
  // copies of K tile j into ring stage sg (all out of range past the end)
  auto issue = [&](int sg, int j) {
    const int64_t k0 = (int64_t)j * SBK;
    const uint32_t kb = (uint32_t)k0 * 2;
    const uint32_t sa = ring_a + (uint32_t)sg * STA, sb = ring_b + (uint32_t)sg * STB;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      copy16(ra, k0 + akc[i] < K ? aoff[i] + kb : kOOB,
             sa + (uint32_t)(wave * (BM / NW) + RPC * i) * ROWB);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      copy16(rb, k0 + bkc[i] < K ? boff[i] + kb : kOOB,
             sb + (uint32_t)(wave * (TBN / NW) + RPC * i) * ROWB);
  };

  // ---- wave sub-tile and its fragment addresses.  Fragment rows are
  // wm*BM/2 + 32*mi + (l%32) (A) and the brow below (B); their swizzle term
  // ((row>>2)&3) is ((l%32)>>2)&3 for all of them.  GATED: wave column wn
  // owns 128/WN gate rows of B and the matching up rows (128 further on).
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lh = lane >> 5;
  const int q = (lr / (16 / CPR)) & (CPR - 1);  // swizzle term of every fragment row
  uint32_t fa[NSUB], fb[NSUB];  // per sub-step s: byte offset of block 0 in a stage of A / B
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const uint32_t ch = (uint32_t)(((2 * s + lh) ^ q) << 4);
    fa[s] = (uint32_t)(wm * (BM / 2) + lr) * ROWB + ch;
    fb[s] = (uint32_t)((GATED ? 128 / WN : 256 / WN) * wn + lr) * ROWB + ch;
  }
  // B block ni starts at row bro(ni) + (128/WN or 256/WN) * wn
  constexpr auto bro = [](int ni) constexpr -> int {
    return GATED ? (ni < NI / 2 ? 0 : 128) + 32 * (ni % (NI / 2)) : 32 * ni;
  };
  auto frags = [&](int sg, int s, u32x4 (&f)[NF]) {
    const unsigned char* sa = ringA + (uint32_t)sg * STA;
    const unsigned char* sb = ringB + (uint32_t)sg * STB;
    // in the order the MFMAs (mi-major) consume them: A0, B0.., A1, A2, ...
    f[0] = *reinterpret_cast<const u32x4*>(sa + fa[s]);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      f[MI + ni] = *reinterpret_cast<const u32x4*>(sb + fb[s] + (uint32_t)bro(ni) * ROWB);
#pragma unroll
    for (int mi = 1; mi < MI; ++mi)
      f[mi] = *reinterpret_cast<const u32x4*>(sa + fa[s] + (uint32_t)(32 * mi) * ROWB);
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
  auto mma = [&](const u32x4 (&f)[NF]) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma32(f[mi], f[MI + ni], acc[mi][ni]);
  };

  const int nk = (int)((K + SBK - 1) / SBK);
  auto next = [](int sg) { return sg + 1 == NST ? 0 : sg + 1; };
  // A wave none of whose rows lies in the group (the last m-tile of a
  // group, or a small group) only moves its share of the copies and keeps
  // the barriers: the same copies, waits and barriers as below, without
  // fragment reads or MFMAs, which leaves its SIMD to the waves that have
  // rows.
  if (__builtin_amdgcn_readfirstlane(wm * (BM / 2) >= rows ? 1 : 0)) {
#pragma unroll
    for (int t = 0; t < NST; ++t) issue(t, t);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NST - 1) * (AI + BI)) : "memory");
    __builtin_amdgcn_s_barrier();
    int s_id = 0;
    for (int j = 0; j < nk; ++j) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NST - 2) * (AI + BI)) : "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(s_id, j + NST);
      s_id = next(s_id);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;  // no row of this wave to write
  }
  u32x4 f0[NF], f1[NF];
  // tiles 0 .. NST-1 into stages 0 .. NST-1; wait for tile 0
#pragma unroll
  for (int t = 0; t < NST; ++t) issue(t, t);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NST - 1) * (AI + BI)) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  frags(0, 0, f0);
  int s_rd = 0;  // stage of tile j
  for (int j = 0; j < nk; ++j) {
    const int s_nx = next(s_rd);  // stage of tile j+1
    // sub-steps 0 .. NSUB-2 of tile j, reading the next sub-step's
    // fragments meanwhile (f0 / f1 alternate)
#pragma unroll
    for (int s = 0; s + 1 < NSUB; ++s) {
      if (s % 2 == 0) {
        frags(s_rd, s + 1, f1);
        mma(f0);
      } else {
        frags(s_rd, s + 1, f0);
        mma(f1);
      }
      sched_spread<MI * NI, NF, kSchedDsRead, 0, kSchedVmem>(
          std::make_integer_sequence<int, MI * NI>{});
    }
    // tile j+1 has landed (this wave's copies, then everyone's: a plain
    // s_barrier, since __syncthreads()'s release fence would wait for all
    // copies), and every wave's reads of tile j are complete (lgkmcnt(0)
    // before the barrier), so tile j's stage can be refilled
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((NST - 2) * (AI + BI)) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // last sub-step of tile j; copy tile j+NST into tile j's stage (first:
    // the copies are the long pole) and read the fragments of tile j+1's
    // sub-step 0
    constexpr bool odd = (NSUB - 1) % 2 == 1;
    if constexpr (odd) {
      issue(s_rd, j + NST);
      frags(s_nx, 0, f0);
      mma(f1);
    } else {
      issue(s_rd, j + NST);
      frags(s_nx, 0, f1);
      mma(f0);
    }
    sched_spread<MI * NI, AI + BI, kSchedVmem, NF, kSchedDsRead>(
        std::make_integer_sequence<int, MI * NI>{});
    if constexpr (!odd) {
      // f0 must hold the next tile's sub-step 0
#pragma unroll
      for (int i = 0; i < NF; ++i) f0[i] = f1[i];
    }
    s_rd = s_nx;
  }
  // drain the copies still in flight before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: lane holds D[8*(e/4) + 4*lh + (e%4)][lr] of each 32x32 block
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = wm * (BM / 2) + mi * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
      if (r >= rows) continue;
      bf16_t* orow = out + (row_begin + r) * N;
      if constexpr (PRE) {
        float* hrow = (float*)out_v + (row_begin + r) * 2 * N;
#pragma unroll
        for (int ni = 0; ni < NI / 2; ++ni) {
          const int64_t c = n0 + (128 / WN) * wn + 32 * ni + lr;
          if (c < N) {
            hrow[c] = acc[mi][ni][e];
            hrow[N + c] = acc[mi][ni + NI / 2][e];
          }
        }
      } else if constexpr (GATED) {
#pragma unroll
        for (int ni = 0; ni < NI / 2; ++ni) {
          const int64_t c = n0 + (128 / WN) * wn + 32 * ni + lr;
          if (c < N)
            orow[c] = f32_to_bf16(swiglu(acc[mi][ni][e], acc[mi][ni + NI / 2][e]));
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int64_t c = n0 + (256 / WN) * wn + 32 * ni + lr;
          if (c < N) orow[c] = f32_to_bf16(acc[mi][ni][e]);
        }
      }
    }
  }
}

// ============================================================ panel_gemm
// bf16, expert groups of at most BM rows with long K (many experts with a
// balanced router, e.g. 256 experts of ~128 rows), where each expert's
// weights are read from HBM once and used by few rows.  Only the token rows
// go through LDS; the weight rows are loaded straight into the MFMA's B
// operand registers, D K tiles ahead of their use, so the LDS holds a deeper
// ring of token rows and no weight tile.
//
// Block tile: BM rows x 256 weight rows, 8 waves in a 1 x 8 grid.  Wave w
// owns 32 weight rows as two 16-row column blocks (gate_up: 16 gate rows and
// the 16 matching up rows, so SwiGLU pairs the two accumulators of a lane;
// down: 32 consecutive rows) and the tile's rows as MIL row blocks of
// v_mfma_f32_16x16x32_bf16 (MIL chosen per tile from its row count, so no
// MFMA, fragment read or copy is spent on 16-row blocks past the group).
// Every A fragment read from LDS feeds two MFMAs.
//
// K tiles of 64: the token rows of tile j are copied global -> LDS into
// stage j % NST of the ring (XOR-swizzled as in tiled_gemm); the weight
// chunks of tile j go to register slot j % D.  Per wave and tile: AI
// copies, then 4 weight loads, all issued at iteration j - D, so one wait
// for vmcnt <= (D-1)*(AI+4) covers both, and a barrier covers the other
// waves' copies.  Tile lookup and tile order: as tiled_gemm.
template <bool GATED, int BM, int NST, int MIL>
__device__ __forceinline__ void panel_tile(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_slot,
    const bf16_t* __restrict__ W, bf16_t* __restrict__ out, int64_t K, int64_t N, int64_t T,
    int64_t Tk, int64_t k, int g, int nt, int64_t row_begin, int rows,
    unsigned char* __restrict__ ringA) {
  constexpr int NW = 8;
  constexpr int SBK = 64, CPR = 8, RPC = 8;
  constexpr uint32_t ROWB = SBK * 2;     // bytes per LDS row
  constexpr int AI = (MIL + 3) / 4;      // A copies (1 KB) per wave per stage
  constexpr int MI = MIL;                // live 16-row blocks (16*MIL >= rows)
  constexpr int D = NST - 1;             // K tiles of weights loaded ahead
  constexpr int BL = 4;                  // weight loads per wave per K tile
  constexpr uint32_t STA = BM * ROWB;    // bytes per stage
  static_assert(RPC * NW * AI <= BM && MIL * 16 <= BM, "copy plan");
  static_assert(D >= 1 && (D - 1) * (AI + BL) < 64, "vmcnt range");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t Kb = (uint32_t)(K * 2);

  const bf16_t* abase = GATED ? A : A + row_begin * K;
  const uint32_t a_bytes = GATED ? (uint32_t)(T * K * 2) : (uint32_t)rows * Kb;
  const int64_t wrows = GATED ? 2 * N : N;
  const bf16_t* bbase = W + (int64_t)g * wrows * K;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)abase, 0, (int)a_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)bbase, 0, (int)(uint32_t)(wrows * K * 2),
                                        kRsrcWord3);

  // ---- token-row copies of the 16*MIL rows the MFMAs read: copy c = 8*i + w
  // (wave w, i < AI) fills rows 8c .. 8c+7 of a stage (1 KB); lane l lands on
  // row 8c + l/8, physical chunk l%8, which holds logical chunk
  // (l%8) ^ ((row/2) & 7)
  const int lrow = lane / CPR;
  uint32_t aoff[AI];
  int akc[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = RPC * (i * NW + wave) + lrow;
    akc[i] = ((lane % CPR) ^ ((r >> 1) & (CPR - 1))) * 8;
    uint32_t o = kOOB;
    if (r < rows) {
      const int64_t src_row =
          GATED ? row_token(row_begin + r, sorted_slot, Tk, k, T) : (int64_t)r;
      o = (uint32_t)src_row * Kb + (uint32_t)akc[i] * 2;
    }
    aoff[i] = o;
  }
  uint32_t ring_a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ringA;
  asm("" : "+s"(ring_a));
  auto issue_a = [&](int j) {
    const int64_t k0 = (int64_t)j * SBK;
    const uint32_t sa = ring_a + (uint32_t)(j % NST) * STA;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      copy16(ra, k0 + akc[i] < K ? aoff[i] + (uint32_t)k0 * 2 : kOOB,
             sa + (uint32_t)(RPC * (i * NW + wave)) * ROWB);
  };

  // ---- weight rows of the wave's two column blocks: lane l loads row l%16
  // of each, K elements 8*(l/16) .. +8 of every 32-wide sub-step (the MFMA's
  // B operand layout)
  const int j16 = lane & 15, kq = lane >> 4;
  uint32_t boff[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t c = GATED ? (int64_t)nt * 128 + 16 * wave + j16
                            : (int64_t)nt * 256 + 32 * wave + 16 * b + j16;
    uint32_t o = kOOB;
    if (c < N) {
      const int64_t wr = GATED ? (b == 0 ? c : N + c) : c;
      o = (uint32_t)wr * Kb + (uint32_t)kq * 16;
    }
    boff[b] = o;
  }
  u32x4 breg[D][2][2];  // [slot][sub-step][block]
  auto issue_b = [&](int j, u32x4 (&dst)[2][2]) {
    const int64_t k0 = (int64_t)j * SBK;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // past K: the offset gets the out-of-range bit (offsets are below 2^31)
      const uint32_t oob = k0 + 32 * s + 8 * kq < K ? 0u : kOOB;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint32_t o = (boff[b] + (uint32_t)(k0 + 32 * s) * 2) | oob;
        asm("" : "+v"(o));  // one load with a computed offset, not a branch
        dst[s][b] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)o, 0, 0));
      }
    }
  };

  // ---- A fragment of row block mi, sub-step s: row 16*mi + l%16, logical
  // chunk 4*s + l/16; the swizzle term ((row/2) & 7) is (l%16)/2 for all mi
  uint32_t fa[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
    fa[s] = (uint32_t)j16 * ROWB + (uint32_t)(((4 * s + kq) ^ (j16 >> 1)) << 4);

  f32x4 acc0[MI], acc1[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    acc0[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nk = (int)((K + SBK - 1) / SBK);
  // tiles 0 .. D-1: copies into stages 0 .. D-1, weights into slots 0 .. D-1,
  // in tile order (the waits below count on it)
#pragma unroll
  for (int t = 0; t < D; ++t) {
    issue_a(t);
    issue_b(t, breg[t]);
    asm volatile("" ::: "memory");
  }
  // one K tile: tile j's weights are in register slot bs
  auto step = [&](int j, u32x4 (&bs)[2][2]) {
    // this wave's copies and loads of tile j are done, then everyone's
    // copies; every wave finished reading tile j-1's stage (its fragments
    // fed the MFMAs of the previous step), which is refilled next
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((D - 1) * (AI + BL)) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue_a(j + D);  // stage (j + D) % NST = (j - 1) % NST; past the end: no data
    const unsigned char* st = ringA + (uint32_t)(j % NST) * STA;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 af[MI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        af[mi] = *reinterpret_cast<const u32x4*>(st + fa[s] + mi * 16 * ROWB);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        acc0[mi] = mfma16(af[mi], bs[s][0], acc0[mi]);
        acc1[mi] = mfma16(af[mi], bs[s][1], acc1[mi]);
      }
    }
    issue_b(j + D, bs);  // the same slot, for tile j + D
  };
  // whole rounds of D tiles (slot u holds tile j0 + u), then the rest: the
  // loop has no exit between its steps, so the compiler's own waits for the
  // weight registers count every load issued since (a partial round inside
  // the loop would make it wait for nearly all of them)
  int j0 = 0;
  for (; j0 + D <= nk; j0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) step(j0 + u, breg[u]);
  }
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (j0 + u < nk) step(j0 + u, breg[u]);
  // drain the loads still in flight before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: lane holds D[4*(l/16) + q][l%16] of each 16x16 block
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * mi + 4 * kq + q;
      if (r >= rows) continue;
      bf16_t* orow = out + (row_begin + r) * N;
      if constexpr (GATED) {
        const int64_t c = (int64_t)nt * 128 + 16 * wave + j16;
        if (c < N) orow[c] = f32_to_bf16(swiglu(acc0[mi][q], acc1[mi][q]));
      } else {
        const int64_t c0 = (int64_t)nt * 256 + 32 * wave + j16;
        if (c0 < N) orow[c0] = f32_to_bf16(acc0[mi][q]);
        if (c0 + 16 < N) orow[c0 + 16] = f32_to_bf16(acc1[mi][q]);
      }
    }
  }
}

// The kernel: tile lookup, then the tile with as many 16-row blocks as its
// rows need (BM/2, 2BM/3, 5BM/6 or BM rows), so that no MFMA or fragment
// read of a block past the group's rows is issued and the K loop stays
// free of branches.
template <bool GATED, int BM, int NST>
__global__ __launch_bounds__(512, 1) void panel_gemm_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ W,
    bf16_t* __restrict__ out, int64_t K, int64_t N, int64_t T, int64_t Tk, int64_t k, int G,
    int ntN) {
  constexpr int MI = BM / 16;
  static_assert(MI % 6 == 0, "row-block split");
  static_assert(NST * BM * 128 <= 160 * 1024, "ring fits the LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char ringA[NST * BM * 128];
  __shared__ int s_tile[3 + 8];
  int g, mt, nt;
  if (!find_tile<8>(offsets, G, BM, ntN, (int)blockIdx.x, &g, &mt, &nt, s_tile)) return;
  const int64_t row_begin = offsets[g] + (int64_t)mt * BM;
  const int64_t rows_left = offsets[g + 1] - row_begin;
  const int rows = (int)(rows_left < BM ? rows_left : BM);
  const int nb = __builtin_amdgcn_readfirstlane((rows + 15) / 16);
  if (nb <= MI / 2)
    panel_tile<GATED, BM, NST, MI / 2>(A, sorted_slot, W, out, K, N, T, Tk, k, g, nt, row_begin,
                                        rows, ringA);
  else if (nb <= 2 * MI / 3)
    panel_tile<GATED, BM, NST, 2 * MI / 3>(A, sorted_slot, W, out, K, N, T, Tk, k, g, nt,
                                            row_begin, rows, ringA);
  else if (nb <= 5 * MI / 6)
    panel_tile<GATED, BM, NST, 5 * MI / 6>(A, sorted_slot, W, out, K, N, T, Tk, k, g, nt,
                                            row_begin, rows, ringA);
  else
    panel_tile<GATED, BM, NST, MI>(A, sorted_slot, W, out, K, N, T, Tk, k, g, nt, row_begin,
                                    rows, ringA);
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

template <bool GATED, bool PRE = false>
hipError_t launch_bf16(const Shape& s, const void* A, const int32_t* sorted_slot,
                       const int32_t* offsets, const void* W, void* out, int64_t K,
                       int64_t N, hipStream_t st) {
  const int G = (int)s.G();
  if (!PRE && s.T <= 64)
    return launch_stream_gemm(GATED, s, A, sorted_slot, offsets, W, out, K, N, st);
  // Tile shapes, as measured fastest on the MI355X:
  //  - large groups (>= 512 rows on average): 256 x 256 tiles, 8 waves (two
  //    per SIMD, so one computes while the other waits), K tiles of 64
  //    (whole 128-byte lines per copied row) in 2 stages of 64 KB;
  //  - routed groups of 112-168 rows on average (balanced routers with many
  //    experts): 192-row tiles, so that a group rarely spills a few rows
  //    into a second m-tile that would read the weight panel again
  //    (DeepSeek-V3 shape: gate_up 3.64 -> 3.54 ms), in panel_gemm (weights
  //    into registers 3 K tiles ahead, only the token rows through LDS:
  //    gate_up 3.48 -> 3.42 ms, down 2.01 -> 1.97 ms); the backward's
  //    pre-activation recompute keeps the 192 x 256 tiled_gemm form;
  //  - other small groups, gate_up: 128 x 256 tiles, 8 waves, K tiles of
  //    64, 3 stages; down: 128 x 256 tiles, 8 waves, K tiles of 32, two
  //    workgroups per CU with 3 stages each (fine-grained Zipf shape: down
  //    199 -> 191 us against 4 waves; the gate_up with two workgroups per
  //    CU, 4 or 8 waves, measured no faster, 64-row tiles 28% slower).
  const int64_t avg_rows = s.R() / (s.G() > 0 ? s.G() : 1);
  const int64_t routed_mean = s.Tk() / s.E;
  const int64_t ncols = GATED ? TBN / 2 : TBN;
  const int ntN = (int)((N + ncols - 1) / ncols);
#define MOE_TILED(bm, nst, occ, nw, sbk)                                                 \
  hipLaunchKernelGGL((tiled_gemm_kernel<GATED, bm, nst, occ, nw, sbk, PRE>),            \
                     dim3(((mtile_bound(s, bm) * (unsigned)ntN) + 7u) & ~7u), dim3(64 * nw), \
                     0, st, (const bf16_t*)A, sorted_slot, offsets, (const bf16_t*)W, out,  \
                     K, N, s.T, s.Tk(), s.k, G, ntN)
  if (avg_rows >= 512) {
    MOE_TILED(256, 2, 1, 8, 64);
  } else if (routed_mean > 112 && routed_mean <= 168) {
    if constexpr (!PRE) {
      hipLaunchKernelGGL((panel_gemm_kernel<GATED, 192, MOE_PANEL_NST>),
                         dim3(((mtile_bound(s, 192) * (unsigned)ntN) + 7u) & ~7u), dim3(512),
                         0, st, (const bf16_t*)A, sorted_slot, offsets, (const bf16_t*)W,
                         (bf16_t*)out, K, N, s.T, s.Tk(), s.k, G, ntN);
    } else {
      MOE_TILED(192, 2, 1, 8, 64);
    }
  } else if (GATED) {
    MOE_TILED(128, 3, 1, 8, 64);
  } else {
    MOE_TILED(128, 3, 2, 8, 32);
  }
#undef MOE_TILED
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

hipError_t launch_gate_up_preact(const Shape& s, const void* x, const int32_t* sorted_slot,
                                 const int32_t* offsets, const void* W_gate_up, float* H,
                                 hipStream_t st) {
  if (s.R() == 0) return hipSuccess;
  if (s.T <= 64) return launch_stream_gate_up_preact(s, x, sorted_slot, offsets, W_gate_up, H, st);
  return launch_bf16<true, true>(s, x, sorted_slot, offsets, W_gate_up, H, s.d, s.f, st);
}

hipError_t launch_down(const Shape& s, const void* act, const int32_t* offsets,
                       const void* W_down, void* expert_out, hipStream_t st) {
  if (s.R() == 0) return hipSuccess;
  if (s.dt == MOE_DT_BF16)
    return launch_bf16<false>(s, act, nullptr, offsets, W_down, expert_out, s.f, s.d, st);
  return launch_f32<false>(s, act, nullptr, offsets, W_down, expert_out, s.f, s.d, st);
}

}  // namespace moe
