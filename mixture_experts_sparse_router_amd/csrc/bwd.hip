// bwd.hip -- backward pass of the layer: the gradients that grouped-GEMM
// training needs (aitoday "MoEs in Transformers" page, section "Training
// MoEs with Transformers": training standardised on grouped GEMMs).
//
// Chain rule through the forward (y_t = sum_j w_tj O_tj + shared,
// O = Wd_e a, a = silu(g) * u, [g; u] = Wgu_e x_t, w = softmax over the k
// selected logits), for a loss gradient dy, over the forward's own
// permutation (expert groups of rows):
//   1. combine_bwd  dO[r] = w dy_t (shared rows: dy_t), dw_tj = dy_t . O[r];
//      router_dl    dl_tj = w_tj (dw_tj - sum_i w_ti dw_ti)
//   2. H = Xg Wgu_e^T           the forward's tiled gate_up GEMM with a
//                               pre-activation fp32 output (recomputes [g; u])
//   3. dA = dO Wd_e             grouped GEMM over rows, weight [d, f] read as [K, N]
//   4. swiglu_bwd   dH = [dA * u * silu'(g), dA * silu(g)]
//   5. dXp = dH Wgu_e           grouped GEMM over rows, weight [2f, d] read as [K, N]
//   6. dWd_e = dO^T A           grouped GEMM over the group's rows as K
//   7. dWgu_e = dH^T Xg         same, token rows gathered
//   8. router_wgrad dWr_e = sum_r dl_r x_t(r), db_e = sum_r dl_r over e's group
//                   and e's copies dropped by a capacity (row chunks, then a
//                   fixed-order sum of the chunks)
//   9. dx_gather    dx_t = sum_j dXp[slot of (t, j)] + shared rows
//                   + sum_j dl_tj Wr_{e_tj}
// With a capacity, a dropped copy (slot_pos < 0) has no row: no expert
// gradient and dw = 0, but its logit keeps dl (the kept weights are not
// renormalised, so every selected logit moves them).
// Gradients come out in fp32; the intermediates dO and dH are rounded to
// bf16 (the GEMM operands), H and dA stay fp32.  Every sum has a fixed
// order (no atomics), so repeated calls are bitwise identical.
//
// The grouped GEMMs share one kernel: 128 x 128 tiles, K tiles of 32 staged
// in LDS (double buffered, the next tile's global loads in registers while
// the current one is multiplied), 4 waves each 64 x 64 with
// v_mfma_f32_32x32x16_bf16.  An operand that is K-contiguous in memory is
// copied to LDS row by row and read as 16-byte fragments of 8 consecutive K
// elements.  One that is contiguous along M or N is copied as it lies (K
// rows of 128 M/N elements) and its fragments are read with gfx950's
// transposing LDS load (ds_read_b64_tr_b16), which hands each lane 4
// consecutive K elements of one M/N column; two of them make a fragment.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kBT = 128;        // tile rows and columns of the 4-wave form
constexpr int kBK = 32;         // K per stage of the 4-wave form
// K-major tile row stride in bf16 for BK K per stage: BK + 8 (80 or 144
// bytes: the 16-byte reads of 16 consecutive rows hit 16 distinct slots)
constexpr int k_row(int BK) { return BK + 8; }
constexpr int kBwdThreads = 256;
// M/N-major tile row stride in bf16 for X columns: X + 32 (a 64-byte shift
// per row: the 8 rows one transposing load touches fall on distinct banks)
constexpr int mn_row(int X) { return X + 32; }
constexpr int tile_elems(int X, int BK) {
  return X * k_row(BK) > BK * mn_row(X) ? X * k_row(BK) : BK * mn_row(X);
}

// Operand tiles in LDS, K-major: [X rows (M or N)][BK] bf16, row stride
// k_row(BK); or M/N-major: [BK K rows][X M or N] bf16, row stride mn_row(X).
template <int BM, int BN, int BK>
struct BwdSmem {
  bf16_t a[2][tile_elems(BM, BK)];
  bf16_t b[2][tile_elems(BN, BK)];
};
// 128 x 128: 40 KB, four workgroups per CU.  The group lookup's scratch
// borrows the start of b[1], which is first written after the lookup's last
// barrier.
static_assert(sizeof(BwdSmem<128, 128, 32>) == 40960, "four workgroups fit one CU's LDS");
static_assert(sizeof(BwdSmem<256, 256, 64>) <= 160 * 1024, "one workgroup fits one CU's LDS");

template <int BK>
__device__ __forceinline__ void store_kc(bf16_t* tile, int row, int kc, const u32x4& v) {
  *reinterpret_cast<u32x4*>(tile + row * k_row(BK) + kc) = v;
}

// Fragment of the 32x32x16 MFMA from an M/N-major tile of row stride RS:
// M/N indices mn .. mn+31, K elements 16 ks .. +15; lane l gets column
// mn + (l % 32), K 8 (l / 32) .. +7 (the layout of a 16-byte K-major
// fragment read).  In each group of 16 lanes (g = l / 16, i = l % 16) the
// transposing load hands lane i element i % 4 of the 8 bytes addressed by
// lane 4q + i / 4 as its element q; so lane i addresses K row r0 + i / 4,
// columns c0 + 4 (i % 4) .. +3, and receives column c0 + i of K rows r0 ..
// r0+3 (a second load: r0+4 .. r0+7), with c0 = mn + 16 (g % 2) and
// r0 = 16 ks + 8 (g / 2).
template <int RS>
__device__ __forceinline__ u32x4 frag_mn(const bf16_t* tile, int mn, int ks, int lane) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const int g = lane >> 4, i = lane & 15;
  const int row = 16 * ks + 8 * (g >> 1) + (i >> 2);
  const int col = mn + 16 * (g & 1) + 4 * (i & 3);
  const bf16_t* p = tile + row * RS + col;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * RS));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return u32x4{a.x, a.y, b.x, b.y};
}

// Which row group (and m-tile) a workgroup owns: group g has
// ceil(n_g / BM) m-tiles.  Cooperative over the workgroup's NW waves
// (4 groups per thread: 256 * NW >= 1024 >= G); sh: 2 + NW ints.
template <int BM, int NW>
__device__ bool find_group_tile(const int32_t* offsets, int G, int tile, int* g_out, int* mt_out,
                                int* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int c[4], mine = 0;
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
  if (lane == 63) sh[2 + wave] = inc;
  if (tid == 0) sh[0] = -1;
  __syncthreads();
  int start = inc - mine;
  for (int w = 0; w < wave; ++w) start += sh[2 + w];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (tile >= start && tile < start + c[i]) {
      sh[0] = tid * 4 + i;
      sh[1] = tile - start;
    }
    start += c[i];
  }
  __syncthreads();
  *g_out = sh[0];
  *mt_out = sh[1];
  const bool ok = sh[0] >= 0;
  __syncthreads();  // sh is reused by the caller's next lookup, if any
  return ok;
}

// ROWS = true:  C[r, n] = sum_k A[src(r), k] B(k, n) over the rows r of each
//   expert group (M = the group's rows, K fixed); A K-contiguous (row
//   src(r) = the token of r when GATHER, else r); B of expert g: B_KC ?
//   B[g][n][k] (K-contiguous) : B[g][k][n] (N-contiguous).  C row r, ldc.
// ROWS = false: C[g][m, n] = sum_{r in group g} A[r, m] B[src(r), n] (K =
//   the group's rows, M and N fixed); A and B contiguous along M and N;
//   C [G][M][N].
// Tile BM x BN (128 or 256 each), one wave per 64 x 64 block of it; BK K
// per stage (32 or 64).
template <bool ROWS, bool B_KC, bool GATHER, int BM = kBT, int BN = kBT, int BK = kBK>
__global__ __launch_bounds__(64 * (BM / 64) * (BN / 64), (BM == 128 && BN == 128) ? 4 : 1)
void bwd_gemm_kernel(
    const bf16_t* __restrict__ A, int64_t lda, const bf16_t* __restrict__ B, int64_t ldb,
    int64_t b_stride, float* __restrict__ C, int64_t ldc, int64_t M, int64_t N, int64_t K,
    const int32_t* __restrict__ offsets, int G, const int32_t* __restrict__ sorted_slot,
    int64_t Tk, int64_t k, int64_t T, int ntM, int ntN) {
  constexpr int WN = BN / 64;               // wave columns
  constexpr int NW = (BM / 64) * WN;        // waves
  constexpr int NT = 64 * NW;               // threads
  constexpr int KC = BK / 8;                // 16-byte chunks per K-major tile row
  constexpr int CA = KC * BM / NT;          // 16-byte chunks of an A tile per thread
  constexpr int CB = KC * BN / NT;          // ... of a B tile
  constexpr int RSA = mn_row(BM), RSB = mn_row(BN), LR = k_row(BK);
  static_assert(CA >= 1 && CB >= 1 && KC * BM % NT == 0 && KC * BN % NT == 0, "staging plan");
  __shared__ __attribute__((aligned(16))) BwdSmem<BM, BN, BK> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int g, mt, nt;
  int64_t row_begin, rows;  // ROWS: the tile's rows; else the group's rows (K)
  if constexpr (ROWS) {
    nt = (int)blockIdx.x % ntN;
    if (!find_group_tile<BM, NW>(offsets, G, (int)blockIdx.x / ntN, &g, &mt,
                                 reinterpret_cast<int*>(sm.b[1])))
      return;
    row_begin = offsets[g] + (int64_t)mt * BM;
    const int64_t left = offsets[g + 1] - row_begin;
    rows = left < BM ? left : BM;
  } else {
    g = (int)blockIdx.x / (ntM * ntN);
    mt = ((int)blockIdx.x / ntN) % ntM;
    nt = (int)blockIdx.x % ntN;
    row_begin = offsets[g];
    rows = offsets[g + 1] - row_begin;
  }
  const int64_t m0 = ROWS ? 0 : (int64_t)mt * BM;
  const int64_t n0 = (int64_t)nt * BN;
  const int64_t KK = ROWS ? K : rows;  // contraction length
  const bf16_t* Bg = B + (ROWS ? (int64_t)g * b_stride : 0);

  // ---- staging plan: thread tid moves chunks c = tid + NT*i of the X*BK/8
  // 16-byte chunks of each operand tile (X = BM for A, BN for B).  K-major
  // tile (ROWS: A, and B when B_KC): tile row c/KC, K elements 8*(c%KC) ..
  // of that row.  M/N-major tile (its global rows are K rows): K row
  // c/(X/8), M/N elements 8*(c%(X/8)) .. of that row.
  constexpr bool A_MN = !ROWS;
  constexpr bool B_MN = ROWS ? !B_KC : true;
  const bf16_t* arow[CA];  // ROWS: A row of the chunk's tile row (null past the tile)
  const bf16_t* brow[CB];  // ROWS && B_KC: B row n of the chunk
  int akc[CA], aro[CA], bkc[CB], bro[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + NT * i;
    aro[i] = c / KC;
    akc[i] = 8 * (c % KC);
    arow[i] = nullptr;
    if constexpr (ROWS) {
      const int r = aro[i];
      if (r < rows) {
        const int64_t grow = row_begin + r;
        const int64_t src = GATHER ? row_token(grow, sorted_slot, Tk, k, T) : grow;
        arow[i] = A + src * lda;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + NT * i;
    bro[i] = c / KC;
    bkc[i] = 8 * (c % KC);
    brow[i] = nullptr;
    if constexpr (ROWS && B_KC) {
      const int64_t n = n0 + bro[i];
      if (n < N) brow[i] = Bg + n * ldb;
    }
  }
  // every load reads a valid address (the group's first row, or the operand's
  // first row, when the chunk lies outside the tile) and is zeroed by a
  // select, so the loads stay unconditional
  const bf16_t* a_safe = ROWS ? A : A + row_begin * lda;
  const bf16_t* b_safe = ROWS ? Bg : B;
  // !ROWS && GATHER: token rows of the B chunks of the next tile to load,
  // looked up one tile ahead so that the row loads do not wait for them
  int32_t tok[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) tok[i] = 0;
  auto tokload = [&](int j) {
    if constexpr (!ROWS && GATHER) {
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int c = tid + NT * i;
        const int64_t kr = (int64_t)j * BK + c / (BN / 8);
        const int64_t rr = row_begin + (kr < KK ? kr : 0);
        tok[i] = (int32_t)row_token(rr, sorted_slot, Tk, k, T);
      }
    }
  };
  u32x4 ra[CA], rb[CB];
  // global loads of K tile j into registers
  auto gload = [&](int j) {
    const int64_t k0 = (int64_t)j * BK;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + NT * i;
      if constexpr (!A_MN) {
        const bool ok = arow[i] != nullptr && k0 + akc[i] < KK;
        ra[i] = zero_unless(ok, ldg16(ok ? arow[i] + k0 + akc[i] : a_safe));
      } else {
        // A[r][m], r the group row row_begin + kr
        const int64_t kr = k0 + c / (BM / 8);
        const int64_t m = m0 + 8 * (c % (BM / 8));
        const bool ok = kr < KK && m < M;
        ra[i] = zero_unless(ok, ldg16(ok ? A + (row_begin + kr) * lda + m : a_safe));
      }
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + NT * i;
      const int64_t kr = k0 + c / (BN / 8);   // M/N-major: the chunk's K row
      const int64_t n = n0 + 8 * (c % (BN / 8));
      if constexpr (!B_MN) {
        const bool ok = brow[i] != nullptr && k0 + bkc[i] < KK;
        rb[i] = zero_unless(ok, ldg16(ok ? brow[i] + k0 + bkc[i] : b_safe));
      } else if constexpr (ROWS) {
        // B[g][k][n]: K row kr
        const bool ok = kr < KK && n < N;
        rb[i] = zero_unless(ok, ldg16(ok ? Bg + kr * ldb + n : b_safe));
      } else {
        // B[src(r)][n], r the group row row_begin + kr
        const bool ok = kr < KK && n < N;
        const int64_t src = GATHER ? (int64_t)tok[i] : row_begin + (ok ? kr : 0);
        rb[i] = zero_unless(ok, ldg16(ok ? B + src * ldb + n : b_safe));
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + NT * i;
      if constexpr (!A_MN) store_kc<BK>(sm.a[buf], aro[i], akc[i], ra[i]);
      else *reinterpret_cast<u32x4*>(sm.a[buf] + (c / (BM / 8)) * RSA + 8 * (c % (BM / 8))) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + NT * i;
      if constexpr (!B_MN) store_kc<BK>(sm.b[buf], bro[i], bkc[i], rb[i]);
      else *reinterpret_cast<u32x4*>(sm.b[buf] + (c / (BN / 8)) * RSB + 8 * (c % (BN / 8))) = rb[i];
    }
  };

  // ---- compute: wave (wm, wn) owns rows wm*64 .. +64 and columns wn*64 ..
  // +64 of the tile, 2 x 2 blocks of 32 x 32
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lh = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;

  const int nk = (int)((KK + BK - 1) / BK);
  if (nk > 0) {
    tokload(0);
    gload(0);
    tokload(1);
    lstore(0);
    __syncthreads();
    for (int j = 0; j < nk; ++j) {
      const int buf = j & 1;
      if (j + 1 < nk) {
        gload(j + 1);
        tokload(j + 2);
      }
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        u32x4 fa[2], fb[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          fa[mi] = A_MN ? frag_mn<RSA>(sm.a[buf], wm * 64 + mi * 32, ks, lane)
                        : *reinterpret_cast<const u32x4*>(
                              sm.a[buf] + (wm * 64 + mi * 32 + lr) * LR + 16 * ks + 8 * lh);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          fb[ni] = B_MN ? frag_mn<RSB>(sm.b[buf], wn * 64 + ni * 32, ks, lane)
                        : *reinterpret_cast<const u32x4*>(
                              sm.b[buf] + (wn * 64 + ni * 32 + lr) * LR + 16 * ks + 8 * lh);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma32(fa[mi], fb[ni], acc[mi][ni]);
      }
      if (j + 1 < nk) lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds D[8*(e/4) + 4*lh + (e%4)][lr] of each block
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rl = wm * 64 + mi * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int64_t n = n0 + wn * 64 + ni * 32 + lr;
        if (n >= N) continue;
        if constexpr (ROWS) {
          if (rl < rows) C[(row_begin + rl) * ldc + n] = acc[mi][ni][e];
        } else {
          const int64_t m = m0 + rl;
          if (m < M) C[((int64_t)g * M + m) * ldc + n] = acc[mi][ni][e];
        }
      }
    }
  }
}

// ------------------------------------------------------------ elementwise

// 1a. One wave per routed copy (t, j): dO row = w dy_t (bf16) and
// dw_tj = dy_t . O_row (each lane takes 8 consecutive elements at a time,
// 16-byte loads, striding over d; then a fixed butterfly); one wave per
// shared row: dO row = dy_t.  d % 8 == 0 and every row is 16-byte aligned.
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const bf16_t* __restrict__ dy, const bf16_t* __restrict__ O,
    const int32_t* __restrict__ slot_pos, const float* __restrict__ topk_w,
    bf16_t* __restrict__ dO, float* __restrict__ dw_out, int64_t T, int64_t d, int64_t k,
    int S) {
  const int lane = threadIdx.x & 63;
  const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // copy, then shared row
  const int64_t Tk = T * k;
  if (c >= Tk + (int64_t)S * T) return;
  if (c >= Tk) {
    const int64_t t = (c - Tk) % T;
    const bf16_t* dyt = dy + t * d;
    bf16_t* dOr = dO + c * d;  // shared rows follow the routed ones in the same order
    for (int64_t i = 8 * lane; i < d; i += 512)
      *reinterpret_cast<u32x4*>(dOr + i) = ldg16(dyt + i);
    return;
  }
  const int64_t t = c / k;
  const int32_t r = slot_pos[c];
  const float w = topk_w[c];
  const bf16_t* dyt = dy + t * d;
  float acc = 0.f;
  if (r >= 0) {
    const bf16_t* Or = O + (int64_t)r * d;
    bf16_t* dOr = dO + (int64_t)r * d;
    for (int64_t i = 8 * lane; i < d; i += 512) {
      const u32x4 gv = ldg16(dyt + i), ov = ldg16(Or + i);
      const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, ow[4] = {ov.x, ov.y, ov.z, ov.w};
      uint32_t res[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float g0 = bf16lo(gw[h]), g1 = bf16hi(gw[h]);
        acc += g0 * bf16lo(ow[h]);
        acc += g1 * bf16hi(ow[h]);
        res[h] = pack_bf16x2(w * g0, w * g1);
      }
      *reinterpret_cast<u32x4*>(dOr + i) = u32x4{res[0], res[1], res[2], res[3]};
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) dw_out[c] = acc;  // dropped copies: 0
}

// 1b. Softmax over the k selected logits: dl_j = w_j (dw_j - sum_i w_i dw_i),
// one thread per token.  A copy dropped by a capacity has dw_j = 0 but its
// weight still enters the normalisation of the kept ones (they are not
// renormalised), so its dl_j = -w_j sum_i w_i dw_i.
__global__ __launch_bounds__(256) void router_dl_kernel(const float* __restrict__ dw,
                                                        const float* __restrict__ topk_w,
                                                        float* __restrict__ dl, int64_t T,
                                                        int64_t k) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  float sw = 0.f;
  for (int64_t j = 0; j < k; ++j) sw += topk_w[t * k + j] * dw[t * k + j];
  for (int64_t j = 0; j < k; ++j) dl[t * k + j] = topk_w[t * k + j] * (dw[t * k + j] - sw);
}

// 4. dH[r, n] = dA * u * silu'(g), dH[r, f + n] = dA * silu(g), from H = [g; u].
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ H,
                                                         const float* __restrict__ dA,
                                                         bf16_t* __restrict__ dH, int64_t R,
                                                         int64_t f) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= R * f) return;
  const int64_t r = i / f, n = i % f;
  const float g = H[r * 2 * f + n], u = H[r * 2 * f + f + n];
  const float da = dA[i];
  const float s = 1.0f / (1.0f + __expf(-g));
  dH[r * 2 * f + n] = f32_to_bf16(da * u * (s * (1.0f + g * (1.0f - s))));
  dH[r * 2 * f + f + n] = f32_to_bf16(da * (g * s));
}

// First dropped row r in [0, D) whose expert key is >= e.  The dropped rows
// hold first the copies with ids outside [0, E) (key -1), then the copies
// over capacity by expert id, so the key never decreases over [0, D).
__device__ __forceinline__ int64_t dropped_lower_bound(const int32_t* __restrict__ topk_idx,
                                                       const int32_t* __restrict__ sorted_slot,
                                                       int64_t D, int e, int E) {
  int64_t lo = 0, hi = D;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    const int32_t id = topk_idx[sorted_slot[mid]];
    const int key = (id >= 0 && id < E) ? id : -1;
    if (key < e) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// 8. Router weight and bias gradients: chunk c of expert e's rows adds
// dl(r) x[t(r)] for its rows in order (8 rows' loads issued together); then
// the chunks are added in order.  Expert e's rows are its group, then the
// copies of e that a capacity dropped (rows in [0, offsets[0]); their dl is
// not zero, see 1b).
__global__ __launch_bounds__(256) void router_wgrad_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ dl,
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ offsets, float* __restrict__ part, float* __restrict__ part_b,
    int64_t d, int64_t k, int E) {
  const int e = blockIdx.x, c = blockIdx.z;
  // four consecutive columns per thread (d % 8 == 0: 8-byte x loads)
  const int64_t col = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4;
  const int64_t colc = col < d ? col : d - 4;
  const int64_t r0 = offsets[e], nk = offsets[e + 1] - r0;
  const int64_t D = offsets[0];
  int64_t dlo = 0, nd = 0;
  if (D > 0) {
    dlo = dropped_lower_bound(topk_idx, sorted_slot, D, e, E);
    nd = dropped_lower_bound(topk_idx, sorted_slot, D, e + 1, E) - dlo;
  }
  // chunk c of the n = nk + nd rows (group rows first, then dropped rows)
  const int64_t n = nk + nd;
  const int64_t per = (n + kRouterChunks - 1) / kRouterChunks;
  const int64_t lo = (int64_t)c * per;
  const int64_t hi = (lo + per < n) ? lo + per : n;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float accb = 0.f;
  // rows base + i for i in [i0, i1), in order
  auto add_rows = [&](int64_t base, int64_t i0, int64_t i1) {
    for (int64_t rb = i0; rb < i1; rb += 8) {
      int32_t slot[8];
      float v[8];
      uint2 xv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) slot[u] = rb + u < i1 ? sorted_slot[base + rb + u] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v[u] = rb + u < i1 ? dl[slot[u]] : 0.f;
        xv[u] = *reinterpret_cast<const uint2*>(
            x + (int64_t)((uint32_t)slot[u] / (uint32_t)k) * d + colc);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc[0] += v[u] * bf16lo(xv[u].x);
        acc[1] += v[u] * bf16hi(xv[u].x);
        acc[2] += v[u] * bf16lo(xv[u].y);
        acc[3] += v[u] * bf16hi(xv[u].y);
        accb += v[u];
      }
    }
  };
  add_rows(r0, lo, hi < nk ? hi : nk);
  if (hi > nk) add_rows(dlo - nk, lo > nk ? lo : nk, hi);
  if (col < d) *reinterpret_cast<f32x4*>(part + ((int64_t)c * E + e) * d + col) = acc;
  if (blockIdx.y == 0 && threadIdx.x == 0) part_b[c * E + e] = accb;
}

__global__ __launch_bounds__(256) void router_wgrad_sum_kernel(const float* __restrict__ part,
                                                               const float* __restrict__ part_b,
                                                               float* __restrict__ dWr,
                                                               float* __restrict__ db, int64_t d,
                                                               int E) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < (int64_t)E * d) {
    float s = 0.f;
    for (int c = 0; c < kRouterChunks; ++c) s += part[(int64_t)c * E * d + i];
    dWr[i] = s;
  }
  if (i < E) {
    float s = 0.f;
    for (int c = 0; c < kRouterChunks; ++c) s += part_b[c * E + i];
    db[i] = s;
  }
}

// 9. dx_t = sum_j dXp[slot_pos(t, j)] + sum_s dXp[T*k + s*T + t]
//         + sum_j dl_tj Wr[e_tj], in that order.  Each thread owns 4
// consecutive elements (d % 8 == 0; dXp, Wr and dx rows 16- or 8-byte
// aligned), and the rows of up to 8 copies are loaded before they are added.
__global__ __launch_bounds__(256) void dx_gather_kernel(
    const float* __restrict__ dXp, const int32_t* __restrict__ slot_pos,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ dl,
    const bf16_t* __restrict__ Wr, float* __restrict__ dx, int64_t T, int64_t d, int k, int S,
    int E) {
  const int64_t t = blockIdx.x;
  const int64_t i = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4;
  if (i >= d) return;
  const int64_t Tk = T * k;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += 8) {
    f32x4 v[8];
    bool ok[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int32_t r = j0 + u < k ? slot_pos[t * k + j0 + u] : -1;
      ok[u] = r >= 0;
      v[u] = ok[u] ? *reinterpret_cast<const f32x4*>(dXp + (int64_t)r * d + i)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (ok[u]) acc += v[u];
  }
  for (int s = 0; s < S; ++s)
    acc += *reinterpret_cast<const f32x4*>(dXp + (Tk + (int64_t)s * T + t) * d + i);
  for (int j = 0; j < k; ++j) {
    const int32_t e = topk_idx[t * k + j];
    if (e >= 0 && e < E) {
      const float w = dl[t * k + j];
      const uint2 b = *reinterpret_cast<const uint2*>(Wr + (int64_t)e * d + i);
      acc[0] += w * bf16lo(b.x);
      acc[1] += w * bf16hi(b.x);
      acc[2] += w * bf16lo(b.y);
      acc[3] += w * bf16hi(b.y);
    }
  }
  *reinterpret_cast<f32x4*>(dx + t * d + i) = acc;
}

inline unsigned tiles_bound(const Shape& s, int BM) {
  const int64_t R = s.R();
  const int64_t nonempty = s.G() < R ? s.G() : R;
  return (unsigned)(R / BM + nonempty + 1);
}

// K per stage of the 16-wave form (Mixtral-shaped backward 21.7 -> 20.8 ms against 32)
constexpr int kBKBig = 64;
// The four expert GEMMs of the backward pass: the two over a group's rows
// with BM x BN tiles, the two weight gradients with WM x WN tiles.
template <int BM, int BN, int WM, int WN>
void launch_bwd_gemms(const Shape& s, const bf16_t* dO, const bf16_t* Wd, const bf16_t* Wgu,
                      bf16_t* dH, const bf16_t* act, const bf16_t* xb, const int32_t* offsets,
                      const int32_t* sorted_slot, float* dA, float* dXp, float* dWd, float* dWgu,
                      const float* H, hipStream_t st) {
  const int G = (int)s.G();
  const int64_t R = s.R(), d = s.d, f = s.f;
  constexpr int NT = 64 * (BM / 64) * (BN / 64), NTW = 64 * (WM / 64) * (WN / 64);
  const unsigned mt = tiles_bound(s, BM);
  auto ntn = [](int64_t n) { return (int)((n + BN - 1) / BN); };
  auto wtm = [](int64_t n) { return (int)((n + WM - 1) / WM); };
  auto wtn = [](int64_t n) { return (int)((n + WN - 1) / WN); };
  constexpr int BK = BM > 128 ? kBKBig : kBK, WK = WM > 128 ? kBKBig : kBK;
  // 3. dA = dO Wd_e: rows, B N-contiguous (Wd_e [d][f] read as [K = d][N = f])
  hipLaunchKernelGGL((bwd_gemm_kernel<true, false, false, BM, BN, BK>), dim3(mt * ntn(f)),
                     dim3(NT), 0, st, dO, d, Wd, f, d * f, dA, f, (int64_t)0, f, d, offsets, G,
                     sorted_slot, s.Tk(), s.k, s.T, 1, ntn(f));
  // 4
  if (R > 0)
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((R * f + 255) / 256)), dim3(256), 0,
                       st, H, (const float*)dA, dH, R, f);
  // 5. dXp = dH Wgu_e: rows, B N-contiguous (Wgu_e [2f][d] read as [K = 2f][N = d])
  hipLaunchKernelGGL((bwd_gemm_kernel<true, false, false, BM, BN, BK>), dim3(mt * ntn(d)),
                     dim3(NT), 0, st, dH, 2 * f, Wgu, d, 2 * f * d, dXp, d, (int64_t)0, d, 2 * f,
                     offsets, G, sorted_slot, s.Tk(), s.k, s.T, 1, ntn(d));
  // 6. dWd_e = dO^T A: K = the group's rows; M = d, N = f
  hipLaunchKernelGGL((bwd_gemm_kernel<false, false, false, WM, WN, WK>),
                     dim3((unsigned)(G * wtm(d) * wtn(f))), dim3(NTW), 0, st, dO, d, act, f,
                     (int64_t)0, dWd, f, d, f, (int64_t)0, offsets, G, sorted_slot, s.Tk(), s.k,
                     s.T, wtm(d), wtn(f));
  // 7. dWgu_e = dH^T Xg: M = 2f, N = d, token rows gathered
  hipLaunchKernelGGL((bwd_gemm_kernel<false, false, true, WM, WN, WK>),
                     dim3((unsigned)(G * wtm(2 * f) * wtn(d))), dim3(NTW), 0, st, dH, 2 * f, xb,
                     d, (int64_t)0, dWgu, d, 2 * f, d, (int64_t)0, offsets, G, sorted_slot,
                     s.Tk(), s.k, s.T, wtm(2 * f), wtn(d));
}

}  // namespace

hipError_t launch_backward(const Shape& s, const void* x, const void* W_router,
                           const void* W_gate_up, const void* W_down, const void* dy,
                           const int32_t* topk_idx, const float* topk_w,
                           const int32_t* offsets, const int32_t* sorted_slot,
                           const int32_t* slot_pos, const void* act, const void* expert_out,
                           float* dx, float* dWr, float* db, float* dWgu, float* dWd, float* dw,
                           void* workspace, hipStream_t st) {
  size_t off[7];
  bwd_layout(s, off);
  char* ws = (char*)workspace;
  bf16_t* dO = (bf16_t*)(ws + off[0]);
  float* H = (float*)(ws + off[1]);
  float* dA = (float*)(ws + off[2]);
  bf16_t* dH = (bf16_t*)(ws + off[3]);
  float* dXp = (float*)(ws + off[4]);
  float* dl = (float*)(ws + off[5]);
  float* part = (float*)(ws + off[6]);
  float* part_b = part + (size_t)kRouterChunks * s.E * s.d;
  const int G = (int)s.G();
  const int64_t R = s.R(), d = s.d, f = s.f;
  const bf16_t* xb = (const bf16_t*)x;
  const bf16_t* Wgu = (const bf16_t*)W_gate_up;
  const bf16_t* Wd = (const bf16_t*)W_down;

  // 1 (no tokens: the weight gradients below still come out, as zeros)
  if (s.T > 0) {
    const int64_t rows1 = s.Tk() + s.S * s.T;
    // dw goes to the caller's array, else to the dl slot (overwritten next)
    float* dwp = dw ? dw : dl;
    hipLaunchKernelGGL(combine_bwd_kernel, dim3((unsigned)((rows1 + 3) / 4)), dim3(256), 0, st,
                       (const bf16_t*)dy, (const bf16_t*)expert_out, slot_pos, topk_w, dO, dwp,
                       s.T, d, s.k, (int)s.S);
    hipLaunchKernelGGL(router_dl_kernel, dim3((unsigned)((s.T + 255) / 256)), dim3(256), 0, st,
                       (const float*)dwp, topk_w, dl, s.T, s.k);
  }
  // 3-7. the expert GEMMs (H = Xg Wgu_e^T first: the forward's tiled gate_up
  // GEMM with a pre-activation output)
  {
    const hipError_t e = launch_gate_up_preact(s, x, sorted_slot, offsets, W_gate_up, H, st);
    if (e != hipSuccess) return e;
  }
  // Tiles (Mixtral-, DeepSeek-, Zipf-shaped backward passes, HIP events): 256 x 256
  // for every GEMM when the groups hold 512+ rows on average (Mixtral 22.5 ->
  // 21.6 ms); else 128 x 128 for the GEMMs over a group's rows and 256 x 256
  // for the weight gradients (DeepSeek 26.2 -> 24.7 ms, Zipf 2.49 -> 2.45 ms),
  // except at decode sizes, where the weight gradients (a few rows of K, fp32
  // outputs) are fastest with 128 x 128 (1.23 against 1.26 ms).
  if (G > 0 && R / G >= 512)
    launch_bwd_gemms<256, 256, 256, 256>(s, dO, Wd, Wgu, dH, (const bf16_t*)act, xb, offsets,
                                         sorted_slot, dA, dXp, dWd, dWgu, H, st);
  else if (s.T > 64)
    launch_bwd_gemms<kBT, kBT, 256, 256>(s, dO, Wd, Wgu, dH, (const bf16_t*)act, xb, offsets,
                                         sorted_slot, dA, dXp, dWd, dWgu, H, st);
  else
    launch_bwd_gemms<kBT, kBT, kBT, kBT>(s, dO, Wd, Wgu, dH, (const bf16_t*)act, xb, offsets,
                                         sorted_slot, dA, dXp, dWd, dWgu, H, st);
  // 8
  hipLaunchKernelGGL(router_wgrad_kernel, dim3((unsigned)s.E, (unsigned)((d + 1023) / 1024),
                                               kRouterChunks),
                     dim3(256), 0, st, xb, (const float*)dl, topk_idx, sorted_slot, offsets, part,
                     part_b, d, s.k, (int)s.E);
  hipLaunchKernelGGL(router_wgrad_sum_kernel, dim3((unsigned)((s.E * d + 255) / 256)), dim3(256),
                     0, st, (const float*)part, (const float*)part_b, dWr, db, d, (int)s.E);
  // 9
  if (s.T > 0)
    hipLaunchKernelGGL(dx_gather_kernel, dim3((unsigned)s.T, (unsigned)((d + 1023) / 1024)),
                       dim3(256), 0, st,
                     (const float*)dXp, slot_pos, topk_idx, (const float*)dl,
                     (const bf16_t*)W_router, dx, s.T, d, (int)s.k, (int)s.S, (int)s.E);
  return hipGetLastError();
}

}  // namespace moe
