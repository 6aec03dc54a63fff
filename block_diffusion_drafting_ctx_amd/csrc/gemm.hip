// Weight-streaming matrix-core GEMMs for the skinny products of the drafting
// hot path, Y[M, N] = A[M, K] . W[N, K]^T, and the kernels that finish them.
//
// The N axis is the concatenation of one or more weight matrices (e.g. W_q |
// W_k | W_v, or W_gate | W_up, or every layer's W_k | W_v), read from the
// context's tiled bf16 copy of them (launch_tile_weights), and is cut into
// tiles of 16 weight rows.  A main kernel produces fp32 partial
// tiles part[k-slice][tile][m][16]; a finish kernel sums the k-slices in a
// fixed order (deterministic) and applies the epilogue of the stage.  Only
// the LM head folds its epilogue (a running argmax) into the main kernel.
//
// Main kernels (gfx950, 64-wide waves, v_mfma_f32_16x16x32_bf16):
//  * gemm_as ("activation stationary", M <= 32): a workgroup copies the
//    activation rows of one k-slice into LDS once, then every wave streams the
//    16 weight rows of its tile for that slice straight from HBM into
//    registers in MFMA operand layout (16 rows x 64 contiguous bytes per load,
//    non-temporal, 8 k-steps per register stage, next stage in flight while
//    the current one feeds the matrix cores).  No barrier in the loop.
//    Measured on MI355X this streams weights at ~5 TB/s where re-reading the
//    activations per wave from L2 halves the rate.
//  * gemm_mt (M > 32, or no gemm_as fit): LDS-tiled 64*MF x 128 blocks,
//    double-buffered 32-deep k stages, optional split-K.
//  * gemm_dma (256-row blocks, bf16 operands): the gemm_mt block with its
//    stages brought into LDS by LDS-DMA loads in MFMA fragment order.
// Activations are a pair of bf16 arrays (hi, lo) with a = hi + lo (two MFMAs
// per fragment); the stages whose outputs do not feed the residual stream
// (context K/V, LM head) use hi only.  RMSNorm is a row scale applied by the
// finish kernel (the product is linear in it): producers store hi/lo of
// (x * gain) plus partial sums of squares of x.
#include "common.h"
#include "kernels.h"

namespace dfl {

// ------------------------------------------------------------------ helpers
// Tiled-weight pointer of lane `lane` of 16-row tile t at column k (k a
// multiple of 32): the lane's 8 columns of row 16t + (lane & 15); the next
// 32 columns of the tile follow 512 elements on.
__device__ __forceinline__ const bf16_t* tile_row_ptr(const GemmArgs& g, int t, int lane, int k) {
  return reinterpret_cast<const bf16_t*>(g.wt) + (((size_t)t * (g.K >> 5) + (k >> 5)) * 64 + lane) * 8;
}

__device__ __forceinline__ float row_rinv(const float* ssq, int nparts, int ld, int m, int kdim, float eps) {
  float s = 0.f;
  for (int p = 0; p < nparts; ++p) s += ssq[p * ld + m];
  return 1.0f / sqrtf(s / (float)kdim + eps);
}

// rinv_out[m] = 1/sqrt(sum_p ssq_in[p][m] / K + eps), computed by the
// workgroups of k-slice 0 after their tiles: chunks of blockDim/16 rows go
// round-robin over those workgroups (index idx of count), 16 lanes per row,
// all partial loads of a lane issued together, fixed summation order.
__device__ void write_rinv(const GemmArgs& g, int idx, int count) {
  const int rows = blockDim.x >> 4;
  for (int r0 = idx * rows; r0 < g.M; r0 += count * rows) {
    const int m = r0 + (threadIdx.x >> 4), part = threadIdx.x & 15;
    float ss = 0.f;
    if (m < g.M) {
      for (int p0 = 0; p0 < g.ssq_nparts; p0 += 256) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int p = p0 + part + 16 * i;
          v[i] = p < g.ssq_nparts ? g.ssq_in[(size_t)p * g.ld_ssq + m] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) ss += v[i];
      }
    }
    ss += __shfl_xor(ss, 8);
    ss += __shfl_xor(ss, 4);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 1);
    if (part == 0 && m < g.M) g.rinv_out[m] = 1.0f / sqrtf(ss / (float)g.K + g.eps);
  }
}

// Packed (value, index) keys of a 16 x 16 MFMA result tile: the largest key per
// activation row m over the tile's 16 columns, valid in every lane after the
// cross-group reduction.
__device__ __forceinline__ uint64_t tile_row_best(const f32x4& v, int n0, int lane) {
  uint64_t best = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t k = argmax_key(v[i], (uint32_t)(n0 + 4 * (lane >> 4) + i));
    best = k > best ? k : best;
  }
  uint64_t o = shfl_xor_u64(best, 16);
  best = o > best ? o : best;
  o = shfl_xor_u64(best, 32);
  return o > best ? o : best;
}

// ------------------------------------------------------------------ gemm_as
template <int MR>
struct AsShape {
  static constexpr int MT = 16 * MR;
  static constexpr int U = 8;  // k-steps per register stage (16 rows x 512 contiguous bytes of W)
};

template <typename S, int MR, int SRC, bool LO, int OUT>
__global__ void __launch_bounds__(512) gemm_as_kernel(const GemmArgs g) {
  constexpr int MT = AsShape<MR>::MT;
  constexpr int U = AsShape<MR>::U;
  extern __shared__ __align__(16) bf16_t sa[];  // [LO ? 2 : 1][MT][ksl + 8]
  const int LDSW = g.ksl + 8;
  const int tid = threadIdx.x, lane = tid & 63, nw = blockDim.x >> 6;
  // wave-uniform: keeps the tile addressing on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = blockIdx.y, k0 = ks * g.ksl;
  const int ntiles = g.N >> 4;
  const int t0 = blockIdx.x * g.tpw, t1 = min(ntiles, t0 + g.tpw);
  int tile = t0 + wave;
  const int niter = g.ksl / (32 * U);

  Raw8 wb0[U], wb1[U];
  auto fetch = [&](Raw8(&wb)[U], const bf16_t* p, int it) {
#pragma unroll
    for (int u = 0; u < U; ++u) load_raw8_nt<bf16_t>(wb[u], p + (it * U + u) * 512);
  };
  const bf16_t* wp = tile_row_ptr(g, tile < t1 ? tile : t0, lane, k0);

  // ---- activation slice -> LDS.  Only the M real rows are staged: LDS rows
  // past M feed only the matrix-core outputs of rows past M, which are never
  // stored.  A thread issues the loads of C pieces before storing any of
  // them, so the staging costs one round of memory latency per C pieces, not
  // one per piece.  The first weight stage is fetched once the slice is
  // staged: issued together with the activation loads, the chip-wide weight
  // burst delayed the activations (measured: every product ~1 us slower).
  const int pr = g.ksl / 8;  // 8-element pieces per row
  const int npieces = min(MT, g.M) * pr;
  constexpr int C = 8;
  for (int p0 = 0; p0 < npieces; p0 += C * (int)blockDim.x) {
    Raw8 rh[C], rl[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int p = p0 + i * (int)blockDim.x + tid;
      if (p >= npieces) continue;
      const int m = p / pr, col = (p - m * pr) * 8;
      if constexpr (SRC == SRC_SPLIT) {
        const size_t o = (size_t)m * g.lda + k0 + col;
        rh[i].lo = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(g.a_hi) + o);
        if constexpr (LO) rl[i].lo = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(g.a_lo) + o);
      } else {
        const int kg = k0 + col;
        const int j = kg / g.src_width;
        load_raw8<S>(rh[i], reinterpret_cast<const S*>(g.src[j]) + (size_t)m * g.src_width + (kg - j * g.src_width));
      }
    }
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int p = p0 + i * (int)blockDim.x + tid;
      if (p >= npieces) continue;
      const int row = p / pr, col = (p - row * pr) * 8;
      bf16x8 hv, lv;
      if constexpr (SRC == SRC_SPLIT) {
        hv = __builtin_bit_cast(bf16x8, rh[i].lo);
        if constexpr (LO) lv = __builtin_bit_cast(bf16x8, rl[i].lo);
      } else if constexpr (sizeof(S) == 2) {
        hv = raw_to_bf16x8<S>(rh[i]);
      } else {  // fp32 sources: split on the fly
        float f[8];
        raw_to_f32x8<S>(rh[i], f);
        f32x4 l0, l1;
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = (__bf16)f[e];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          l0[e] = f[e] - (float)hv[e];
          l1[e] = f[4 + e] - (float)hv[4 + e];
        }
        lv = f32x8_to_bf16x8(l0, l1);
      }
      *reinterpret_cast<bf16x8*>(&sa[row * LDSW + col]) = hv;
      if constexpr (LO) *reinterpret_cast<bf16x8*>(&sa[(MT + row) * LDSW + col]) = lv;
    }
  }
  if (tile < t1) fetch(wb0, wp, 0);
  __syncthreads();

  const bf16_t* ah = &sa[(lane & 15) * LDSW + (lane >> 4) * 8];
  const bf16_t* al = &sa[(MT + (lane & 15)) * LDSW + (lane >> 4) * 8];
  uint64_t wbest[MR];  // OUT_ARGMAX: running best key of row 16*mi + (lane & 15) over this wave's tiles
#pragma unroll
  for (int mi = 0; mi < MR; ++mi) wbest[mi] = 0;
  for (; tile < t1; tile += nw) {
    f32x4 acc[MR];
#pragma unroll
    for (int mi = 0; mi < MR; ++mi) acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](Raw8(&wb)[U], int it) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = (it * U + u) * 32;
        const bf16x8 wv = raw_to_bf16x8<bf16_t>(wb[u]);
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) {
          acc[mi] = mfma16x16x32(wv, *reinterpret_cast<const bf16x8*>(ah + 16 * mi * LDSW + kk), acc[mi]);
          if (LO) acc[mi] = mfma16x16x32(wv, *reinterpret_cast<const bf16x8*>(al + 16 * mi * LDSW + kk), acc[mi]);
        }
      }
    };
    const int next = tile + nw;
    const bf16_t* np = tile_row_ptr(g, next < t1 ? next : tile, lane, k0);
    for (int it = 0; it < niter; it += 2) {
      if (it + 1 < niter) fetch(wb1, wp, it + 1);
      else if (next < t1) fetch(wb1, np, 0);
      compute(wb0, it);
      if (it + 1 < niter) {
        if (it + 2 < niter) fetch(wb0, wp, it + 2);
        else if (next < t1) fetch(wb0, np, 0);
        compute(wb1, it + 1);
      }
    }
    if ((niter & 1) && next < t1) {
#pragma unroll
      for (int u = 0; u < U; ++u) wb0[u] = wb1[u];
    }
    wp = np;

    // lane holds Y[m = 16*mi + (lane & 15)][n = 16*tile + 4*(lane >> 4) + i]
#pragma unroll
    for (int mi = 0; mi < MR; ++mi) {
      const int m = 16 * mi + (lane & 15);
      if constexpr (OUT == OUT_PARTIAL) {
        if (m < g.M)
          *reinterpret_cast<f32x4*>(g.part + (((size_t)ks * ntiles + tile) * g.M + m) * 16 + 4 * (lane >> 4)) =
              acc[mi];
      } else {
        const uint64_t best = tile_row_best(acc[mi], tile * 16, lane);
        wbest[mi] = best > wbest[mi] ? best : wbest[mi];
        if (g.logits_dbg != nullptr && m < g.M) {
          const float r = row_rinv(g.ssq_in, g.ssq_nparts, g.ld_ssq, m, g.K, g.eps);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            g.logits_dbg[(size_t)m * g.N + tile * 16 + 4 * (lane >> 4) + i] = acc[mi][i] * r;
        }
      }
    }
  }
  if constexpr (OUT == OUT_ARGMAX) {
    // one key per (workgroup, row): fold the waves' running bests through LDS
    // (the activation slice is no longer read once every wave is past its tiles)
    __syncthreads();
    uint64_t* sb = reinterpret_cast<uint64_t*>(sa);  // [nw][MT]
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int mi = 0; mi < MR; ++mi) sb[wave * MT + 16 * mi + (lane & 15)] = wbest[mi];
    }
    __syncthreads();
    for (int m = tid; m < MT; m += blockDim.x) {
      uint64_t b = sb[m];
      for (int w = 1; w < nw; ++w) b = sb[w * MT + m] > b ? sb[w * MT + m] : b;
      if (m < g.M) g.best_part[(size_t)blockIdx.x * g.ld_best + m] = b;
    }
  }
  if (g.rinv_out != nullptr && blockIdx.y == 0) write_rinv(g, blockIdx.x, gridDim.x);
}

// ------------------------------------------------------------------ gemm_mt
// LDS-tiled product for M > 32 (batched drafting, batched fusion).  A
// workgroup of 8 waves computes a BM x BN block of Y with BM = 64*MF and
// BN = 32*NF: the waves are 4 along M (16*MF rows each) by 2 along N (16*NF
// columns each), so a wave holds NF x MF 16x16 accumulators and reads NF
// weight and MF (x2 for hi/lo) activation fragments per 32-deep k-step.  The
// fragment reads per matrix-core op fall as the wave tile grows.  LDS rows are
// 96 bytes (32 elements + 16 of padding): measured on gfx950, 16-row fragment
// reads at a 96-byte row stride run at ~460 GB/s per compute unit against
// ~265 GB/s at 80 bytes.  K advances in stages of 32 through a double-buffered
// LDS ring; global loads run two stages ahead in registers, issued
// unconditionally (past the last stage the last one is fetched again and
// stored to the idle buffer) so that every path has the same loads in flight
// and the wait before a stage's stores counts only that stage's loads.  One
// barrier per stage.
//
// Blocks are numbered so that the M blocks sharing a weight block are
// dispatched back to back on the same XCD (workgroup L runs on XCD L % 8), so
// the weight block is fetched from HBM once into that XCD's L2.
// Stage depth: 32 at 256-row blocks (matrix-core bound; the two stages and
// their hi/lo activations fill the LDS), 64 at 64- and 128-row blocks, where
// the product streams weights and a 32-deep stage moved too few bytes per
// barrier (the rows are then 160 bytes, also a conflict-free stride).
template <int MF, int NF>
struct MtShape {
  static constexpr int BM = 64 * MF;
  static constexpr int BN = 32 * NF;
  static constexpr int BK = MF >= 4 ? 32 : 64;
  static constexpr int KST = BK / 32;  // 32-deep k-steps per stage
  static constexpr int LDK = BK + 16;  // LDS row stride (elements): 96- or 160-byte rows, conflict-free fragment reads
  static constexpr int APR = BK / 8;   // 8-element activation pieces per row and stage
  static constexpr int APT = (BM * APR + 511) / 512;  // activation pieces per thread per array
  static constexpr int WPT = (BN * 4 * KST + 511) / 512;  // weight pieces (16 bytes) per thread
};

template <int MF, int NF, int SRC, bool LO>
struct MtRegs {
  Raw8 w[MtShape<MF, NF>::WPT];
  Raw8 a[MtShape<MF, NF>::APT];
  Raw8 l[LO && SRC == SRC_SPLIT ? MtShape<MF, NF>::APT : 1];
};

size_t gemm_mt_lds_bytes(int MF, int NF, bool lo) {
  const int BM = 64 * MF, BN = 32 * NF, BK = MF >= 4 ? 32 : 64;
  return (size_t)2 * ((lo ? 2 : 1) * BM + BN) * (BK + 16) * 2;
}

template <typename S, int MF, int NF, int SRC, bool LO, int OUT>
__global__ void __launch_bounds__(512) gemm_mt_kernel(const GemmArgs g) {
  using Sh = MtShape<MF, NF>;
  constexpr int BM = Sh::BM, BN = Sh::BN, BK = Sh::BK, LDK = Sh::LDK, APT = Sh::APT, WPT = Sh::WPT;
  constexpr int KST = Sh::KST, APR = Sh::APR;
  constexpr int NA = LO ? 2 : 1;
  constexpr int STAGE = (NA * BM + BN) * LDK;
  using Regs = MtRegs<MF, NF, SRC, LO>;
  extern __shared__ __align__(16) bf16_t sm[];  // [2][NA*BM + BN][LDK]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2;

  // ---- block -> (n block, m block, k slice)
  const int L = blockIdx.x, xcd = L & 7, slot = L >> 3;
  const int mb = slot % g.nbm;
  const int unit = (slot / g.nbm) * 8 + xcd;
  if (unit >= g.nbn * g.KS) return;  // grid padding
  const int nb = unit % g.nbn, ks = unit / g.nbn;
  const int n0 = nb * BN, m0 = mb * BM;
  const int kbeg = ks * g.kslice, nk = g.kslice / BK;

  // ---- per-thread load sources (fixed rows, k advances).  Weight piece q =
  // tid + 512 i is lane q & 63 of 1 KB block q >> 6 of the stage, block b
  // being k-step b % KST of tile b / KST: 64 threads read one tile's 1 KB
  // k-step block; past N the last tile is re-read (unused).  When the pieces
  // are not a multiple of 512 (NF = 6) a thread with no piece i repeats its
  // piece 0 (same source, same LDS slot), so the loads stay unconditional.
  auto wq = [&](int i) { return tid + i * 512 < BN * 4 * KST ? tid + i * 512 : tid; };
  const bf16_t* wsrc[WPT];
  const int nks = g.K >> 5, ntl = g.N >> 4;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int q = wq(i), b = q >> 6, t = min(n0 / 16 + b / KST, ntl - 1);
    wsrc[i] = reinterpret_cast<const bf16_t*>(g.wt) + (((size_t)t * nks + kbeg / 32 + b % KST) * 64 + (q & 63)) * 8;
  }
  auto wrow = [&](int i) { return (((wq(i) >> 6) / KST) << 4) + (tid & 15); };  // block row of weight piece i
  auto wcol = [&](int i) { return ((wq(i) >> 6) % KST) * 32 + ((tid >> 4) & 3) * 8; };  // and its stage column
  auto prow = [&](int i) { return (tid + i * 512) / APR; };  // row of a thread's i-th activation piece
  const int pc = (tid % APR) * 8;                            // its column within the stage
  auto aok = [&](int i) { return (i + 1) * 512 <= BM * APR || tid + i * 512 < BM * APR; };  // whole pieces: always

  auto gload = [&](Regs& r, int kt) {
    const int k = kbeg + kt * BK;
#pragma unroll
    for (int i = 0; i < WPT; ++i) load_raw8<bf16_t>(r.w[i], wsrc[i] + kt * 512 * KST);
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      if (!aok(i)) continue;
      const int m = min(m0 + prow(i), g.M - 1);
      if constexpr (SRC == SRC_SPLIT) {
        const size_t o = (size_t)m * g.lda + k + pc;
        r.a[i].lo = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(g.a_hi) + o);
        if constexpr (LO) r.l[i].lo = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(g.a_lo) + o);
      } else {
        const int kg = k + pc;
        const int j = kg / g.src_width;
        load_raw8<S>(r.a[i], reinterpret_cast<const S*>(g.src[j]) + (size_t)m * g.src_width + (kg - j * g.src_width));
      }
    }
  };
  // live = false (a stage past the end, three-set pipeline): the weights are
  // stored as zeros by a select, so the stage adds nothing
  auto sstore = [&](const Regs& r, int buf, bool live = true) {
    bf16_t* st = sm + buf * STAGE;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<bf16x8*>(&st[(NA * BM + wrow(i)) * LDK + wcol(i)]) =
          __builtin_bit_cast(bf16x8, live ? r.w[i].lo : z);
    }
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      if (!aok(i)) continue;
      bf16x8 hv, lv;
      if constexpr (SRC == SRC_SPLIT) {
        hv = __builtin_bit_cast(bf16x8, r.a[i].lo);
        if constexpr (LO) lv = __builtin_bit_cast(bf16x8, r.l[i].lo);
      } else if constexpr (sizeof(S) == 2) {
        hv = raw_to_bf16x8<S>(r.a[i]);
      } else {  // fp32 sources: split on the fly
        float f[8];
        raw_to_f32x8<S>(r.a[i], f);
        f32x4 l0, l1;
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = (__bf16)f[e];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          l0[e] = f[e] - (float)hv[e];
          l1[e] = f[4 + e] - (float)hv[4 + e];
        }
        lv = f32x8_to_bf16x8(l0, l1);
      }
      *reinterpret_cast<bf16x8*>(&st[prow(i) * LDK + pc]) = hv;
      if constexpr (LO) *reinterpret_cast<bf16x8*>(&st[(BM + prow(i)) * LDK + pc]) = lv;
    }
  };

  f32x4 acc[NF][MF];
#pragma unroll
  for (int fn = 0; fn < NF; ++fn)
#pragma unroll
    for (int fm = 0; fm < MF; ++fm) acc[fn][fm] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
    const bf16_t* st = sm + buf * STAGE;
#pragma unroll
    for (int kq = 0; kq < KST; ++kq) {
      const int fr = (lane & 15) * LDK + 8 * (lane >> 4) + 32 * kq;
      bf16x8 af[MF], al[MF];
#pragma unroll
      for (int fm = 0; fm < MF; ++fm) {
        af[fm] = *reinterpret_cast<const bf16x8*>(&st[(16 * MF * wm + 16 * fm) * LDK + fr]);
        if constexpr (LO) al[fm] = *reinterpret_cast<const bf16x8*>(&st[(BM + 16 * MF * wm + 16 * fm) * LDK + fr]);
      }
#pragma unroll
      for (int fn = 0; fn < NF; ++fn) {
        const bf16x8 wf = *reinterpret_cast<const bf16x8*>(&st[(NA * BM + 16 * NF * wn + 16 * fn) * LDK + fr]);
#pragma unroll
        for (int fm = 0; fm < MF; ++fm) {
          acc[fn][fm] = mfma16x16x32(wf, af[fm], acc[fn][fm]);
          if constexpr (LO) acc[fn][fm] = mfma16x16x32(wf, al[fm], acc[fn][fm]);
        }
      }
    }
  };

  // ---- pipeline.  256-row blocks (matrix-core bound): registers r0 / r1
  // alternate, loads two stages ahead; the stage count nk is even (the planner
  // splits K into k-slices of a multiple of 64).  64- and 128-row blocks
  // (weight streaming, where a stage's matrix work is short and the loop waits
  // on memory latency): three register sets, loads three stages ahead; the
  // loop runs in threes and a stage past the end is stored with zero weights.
  constexpr bool R3 = MF <= 2;
  Regs r0, r1, r2;
  gload(r0, 0);
  gload(r1, 1);
  if constexpr (R3) gload(r2, min(2, nk - 1));
  sstore(r0, 0);
  __syncthreads();
  // cur: free (its stage kt is in LDS);  nxt: stage kt+1, loaded
  auto step = [&](Regs& cur, Regs& nxt, int kt) {
    gload(cur, min(kt + (R3 ? 3 : 2), nk - 1));
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before the matrix work
    compute(kt & 1);
    sstore(nxt, (kt + 1) & 1, !R3 || kt + 1 < nk);  // after the last stage: into the idle buffer, unused
    __syncthreads();
  };
  if constexpr (R3) {
    for (int kt = 0; kt < nk; kt += 3) {
      step(r0, r1, kt);
      step(r1, r2, kt + 1);
      step(r2, r0, kt + 2);
    }
  } else {
    for (int kt = 0; kt < nk; kt += 2) {
      step(r0, r1, kt);
      step(r1, r0, kt + 1);
    }
  }

  // ---- epilogue.  lane holds Y[m = (lane & 15) + row base][n = 4*(lane >> 4) + i + column base]
  if constexpr (OUT == OUT_PARTIAL) {
    const int ntiles = g.N >> 4;
#pragma unroll
    for (int fn = 0; fn < NF; ++fn) {
      const int n = n0 + 16 * NF * wn + 16 * fn;
      if (n >= g.N) continue;
#pragma unroll
      for (int fm = 0; fm < MF; ++fm) {
        const int m = m0 + 16 * MF * wm + 16 * fm + (lane & 15);
        if (m < g.M)
          *reinterpret_cast<f32x4*>(g.part + (((size_t)ks * ntiles + (n >> 4)) * g.M + m) * 16 + 4 * (lane >> 4)) =
              acc[fn][fm];
      }
    }
    if (g.rinv_out != nullptr && ks == 0) write_rinv(g, nb * g.nbm + mb, g.nbn * g.nbm);
  } else {
    uint64_t* sb = reinterpret_cast<uint64_t*>(sm);  // [2][BM]; the ring is idle after the last barrier
#pragma unroll
    for (int fm = 0; fm < MF; ++fm) {
      uint64_t best = 0;
#pragma unroll
      for (int fn = 0; fn < NF; ++fn) {
        const int n = n0 + 16 * NF * wn + 16 * fn;
        if (n < g.N) {
          const uint64_t t = tile_row_best(acc[fn][fm], n, lane);
          best = t > best ? t : best;
        }
      }
      if ((lane >> 4) == 0) sb[wn * BM + 16 * MF * wm + 16 * fm + (lane & 15)] = best;
    }
    if (g.logits_dbg != nullptr) {
#pragma unroll
      for (int fn = 0; fn < NF; ++fn) {
        const int n = n0 + 16 * NF * wn + 16 * fn;
        if (n >= g.N) continue;
#pragma unroll
        for (int fm = 0; fm < MF; ++fm) {
          const int m = m0 + 16 * MF * wm + 16 * fm + (lane & 15);
          if (m >= g.M) continue;
          const float r = row_rinv(g.ssq_in, g.ssq_nparts, g.ld_ssq, m, g.K, g.eps);
#pragma unroll
          for (int i = 0; i < 4; ++i) g.logits_dbg[(size_t)m * g.N + n + 4 * (lane >> 4) + i] = acc[fn][fm][i] * r;
        }
      }
    }
    __syncthreads();
    for (int rr = tid; rr < BM; rr += 512) {
      const uint64_t a = sb[rr], b = sb[BM + rr];
      if (m0 + rr < g.M) g.best_part[(size_t)nb * g.ld_best + m0 + rr] = a > b ? a : b;
    }
  }
}

// ------------------------------------------------------------------ gemm_dma
// The 256-row tiled product (bf16 operands) with its stages brought into LDS
// by LDS-DMA loads in MFMA fragment order.  A stage is one 32-deep k-step:
// the block's 2*NF weight tiles (the 1 KB k-step blocks of the tiled copy,
// copied as they are) and 16 activation row groups per array (hi, lo), each
// a 1 KB block whose lane l holds row 16g + (l & 15), columns 8(l >> 4) .. + 7
// of the k-step: copied as it is from activations stored in fragment blocks
// (a_blocked; eight whole 128-byte lines per load), else gathered from
// row-major rows (sixteen 64-byte pieces per load).  A fragment is then one
// ds_read_b128 at 16*lane of its block (contiguous across the wave: no bank conflicts, no
// padding), no stage passes through registers, and NS stages are in flight
// (NS - 1 ahead of the one being computed).  Each wave issues the same
// number of block loads for every stage (spare loads repeat the stage's last
// block into its own place), so the wait for a stage is vmcnt((NS-2) * PL),
// PL the loads per wave and stage.
// MF row fragments per wave (4 waves along M): 256-row blocks at MF = 4,
// 192-row blocks at MF = 3, 64- and 128-row blocks (MF = 1, 2) for the fusion.
template <int MF, int NF, bool LO>
struct DmaShape {
  static constexpr int BM = 64 * MF, NT = 2 * NF, NA = LO ? 2 : 1;
  static constexpr int NB = NT + (BM / 16) * NA;   // 1 KB blocks per stage
  static constexpr int PW = (NB + 7) / 8;          // block loads per wave and stage
  static constexpr int SLOT = NB * 1024;
  static constexpr int NS = (160 * 1024 - 4096) / SLOT >= 4 ? 4 : 3;  // stages in the LDS ring
  static_assert(3 * SLOT <= 160 * 1024, "three stages fit the LDS");
};

size_t gemm_dma_lds_bytes(int MF, int NF, bool lo, bool swiglu) {
  const int nb = 2 * NF + 4 * MF * (lo ? 2 : 1);
  const int ns = (160 * 1024 - 4096) / (nb * 1024) >= 4 ? 4 : 3;
  return (size_t)ns * (nb * 1024 + (swiglu ? 2048 : 0));
}

template <int MF, int NF, int SRC, bool LO, int OUT>
__global__ void __launch_bounds__(512) gemm_dma_kernel(const GemmArgs g) {
  using Sh = DmaShape<MF, NF, LO>;
  constexpr int BM = Sh::BM, NT = Sh::NT, NB = Sh::NB, PW = Sh::PW, SLOT = Sh::SLOT, NS = Sh::NS;
  constexpr int AG = BM / 16;  // activation row groups per array
  constexpr bool SW = OUT == OUT_SWIGLU;
  constexpr int PL = PW + (SW ? 1 : 0);  // loads per wave and stage (SW: + the stage's sums of squares)
  // stage operands double-buffered in registers where two sets fit beside the accumulators
  constexpr bool DB = (MF * (LO ? 2 : 1) + NF) * 8 + MF * NF * 4 <= 224;
  static_assert((NS - 2) * PL < 64, "vmcnt range");
  static_assert(!SW || (SRC == SRC_SPLIT && !LO && BM == 256 && NS * SLOT >= 4 * NF * MF * 1024 + 3072),
                "SiLU epilogue: 256-row plain blocks, the exchange fits the ring");
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;

  // ---- block -> (n block, m block, k slice), as in gemm_mt
  const int L = blockIdx.x, xcd = L & 7, slot0 = L >> 3;
  const int mb = slot0 % g.nbm;
  const int unit = (slot0 / g.nbm) * 8 + xcd;
  if (unit >= g.nbn * g.KS) return;  // grid padding
  const int nb = unit % g.nbn, ks = unit / g.nbn;
  const int n0 = nb * (32 * NF), m0 = mb * BM;
  const int kbeg = ks * g.kslice, nk = g.kslice / 32;
  const int nks = g.K >> 5, ntl = g.N >> 4;

  // ---- this wave's block loads of a stage: block b = wave + 8 i (the last
  // block when past the stage).  Weight tile blocks are contiguous 1 KB; an
  // activation block gathers 16 rows (rows past M repeat row M - 1).
  const char* src0[PW];
  int step[PW];  // bytes per k-step of the block's source
  int dst[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int b = min(wave + 8 * i, NB - 1);
    dst[i] = b * 1024;
    if (b < NT) {
      // (SW: the waves of wn = 0 take gate tiles, those of wn = 1 the matching up tiles)
      const int t = SW ? (b < NF ? nb * NF + b : g.up_tile0 + nb * NF + (b - NF)) : min(n0 / 16 + b, ntl - 1);
      src0[i] = reinterpret_cast<const char*>(g.wt) + ((size_t)(t * nks + kbeg / 32) * 64 + lane) * 16;
      step[i] = 1024;
    } else {
      const int a = b - NT, arr = a / AG, grp = a % AG;
      const int m = min(m0 + 16 * grp + (lane & 15), g.M - 1);
      const int k = kbeg + 8 * (lane >> 4);
      step[i] = 64;
      if constexpr (SRC == SRC_SPLIT) {
        const char* base = reinterpret_cast<const char*>(arr ? g.a_lo : g.a_hi);
        if (g.a_blocked) {
          // the group's k-steps are consecutive kilobytes (a last group past M
          // reads the final 16-row block; its rows past M are never stored)
          const int a16 = min(m0 / 16 + grp, (g.M + 15) / 16 - 1);
          src0[i] = base + (((size_t)a16 * (g.K / 32) + kbeg / 32) * 64 + lane) * 16;
          step[i] = 1024;
        } else {
          src0[i] = base + ((size_t)m * g.lda + k) * 2;
        }
      } else {
        src0[i] = nullptr;  // per stage: the source array holding the k-step
      }
    }
  }
  // SW: thread tid sums, one per stage, the K/16 partial sums of squares of
  // row m0 + (tid & 255): half tid >> 8 of them (K/32 = nk stages each).
  // They arrive by a 4-byte LDS-DMA load per wave and stage beside the stage.
  const float* ssq_src = nullptr;
  float ssq_acc = 0.f;
  if constexpr (SW) ssq_src = g.ssq_in + (size_t)((tid >> 8) * nk) * g.ld_ssq + min(m0 + (tid & 255), g.M - 1);
  auto issue = [&](int kt, int s) {
    unsigned char* sl = lds + s * SLOT;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const char* src;
      if constexpr (SRC == SRC_SPLIT) {
        src = src0[i] + (size_t)kt * step[i];
      } else {
        const int b = min(wave + 8 * i, NB - 1);
        if (b < NT) {
          src = src0[i] + (size_t)kt * step[i];
        } else {
          const int grp = (b - NT) % AG;
          const int m = min(m0 + 16 * grp + (lane & 15), g.M - 1);
          const int k = kbeg + 32 * kt;  // one k-step lies in one source (src_width % 32 == 0)
          const int j = k / g.src_width;
          src = reinterpret_cast<const char*>(g.src[j]) +
                ((size_t)m * g.src_width + (k - j * g.src_width) + 8 * (lane >> 4)) * 2;
        }
      }
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(sl + dst[i]), 16, 0, 0);
    }
    if constexpr (SW)
      __builtin_amdgcn_global_load_lds(ssq_src + (size_t)kt * g.ld_ssq,
                                       (lds_void_t*)(lds + NS * SLOT + s * 2048 + wave * 256), 4, 0, 0);
    asm volatile("" ::: "memory");
  };

  f32x4 acc[NF][MF];
#pragma unroll
  for (int fn = 0; fn < NF; ++fn)
#pragma unroll
    for (int fm = 0; fm < MF; ++fm) acc[fn][fm] = f32x4{0.f, 0.f, 0.f, 0.f};
  // A stage's operands in registers: MF activation (x2 for hi/lo) and NF
  // weight fragments, and (SW) this thread's partial sum of squares.
  struct Frags {
    bf16x8 a[MF], l[MF], w[NF];
    float ssq;
  };
  auto read = [&](int s, Frags& f) {
    if constexpr (SW) f.ssq = reinterpret_cast<const float*>(lds + NS * SLOT)[s * 512 + tid];
    const unsigned char* sl = lds + s * SLOT + 16 * lane;
#pragma unroll
    for (int fm = 0; fm < MF; ++fm) {
      f.a[fm] = *reinterpret_cast<const bf16x8*>(sl + (NT + MF * wm + fm) * 1024);
      if constexpr (LO) f.l[fm] = *reinterpret_cast<const bf16x8*>(sl + (NT + AG + MF * wm + fm) * 1024);
    }
#pragma unroll
    for (int fn = 0; fn < NF; ++fn) f.w[fn] = *reinterpret_cast<const bf16x8*>(sl + (NF * wn + fn) * 1024);
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int fn = 0; fn < NF; ++fn) {
#pragma unroll
      for (int fm = 0; fm < MF; ++fm) {
        acc[fn][fm] = mfma16x16x32(f.w[fn], f.a[fm], acc[fn][fm]);
        if constexpr (LO) acc[fn][fm] = mfma16x16x32(f.w[fn], f.l[fm], acc[fn][fm]);
      }
    }
    if constexpr (SW) ssq_acc += f.ssq;
  };
  constexpr int NRD = MF * (LO ? 2 : 1) + NF + (SW ? 1 : 0);  // LDS reads of a stage
  constexpr int NMF = MF * NF * (LO ? 2 : 1);                 // matrix ops of a stage

  // ---- pipeline: NS - 1 stages requested ahead (past the end: the last
  // stage again, into its own slot; never computed)
#pragma unroll
  for (int j = 0; j < NS - 1; ++j) issue(min(j, nk - 1), j);
  if constexpr (DB) {
    // Two register sets: each step reads the next stage's fragments and then
    // runs the current stage's matrix ops, so the reads fly under them.  A
    // slot is refilled once every wave's reads of it are done (lgkmcnt(0)
    // before the barrier), one stage later than when the reads sit in the
    // step that uses them; the ring keeps NS - 1 stages in flight.  Every
    // step has the same loads, waits and reads (the last one reads a slot it
    // never uses): a step without them would make the compiler wait for all
    // reads in flight before the next step's matrix ops.
    Frags f0, f1;
    wait_vm<(NS - 2) * PL>();  // stage 0 is in LDS (every wave's, after the barrier)
    raw_barrier();
    issue(min(NS - 1, nk - 1), NS - 1);
    read(0, f0);
    auto step = [&](int kt, const Frags& cur, Frags& nxt) {
      wait_vm<(NS - 2) * PL>();  // this wave's loads of stage kt + 1 are in LDS
      wait_lgkm0();              // this wave's reads of stage kt are in registers
      raw_barrier();             // ... every wave's: stage kt's slot is free
      issue(min(kt + NS, nk - 1), kt % NS);
      read((kt + 1) % NS, nxt);
      __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);  // the next stage's reads go out first
      mma(cur);
      __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
    };
    for (int kt = 0; kt < nk; kt += 2) {
      step(kt, f0, f1);
      if (kt + 1 < nk) step(kt + 1, f1, f0);
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      wait_vm<(NS - 2) * PL>();  // this wave's loads of stage kt are in LDS
      raw_barrier();             // ... every wave's, and every wave is done with stage kt - 1
      issue(min(kt + NS - 1, nk - 1), (kt + NS - 1) % NS);
      Frags f;
      read(kt % NS, f);
      // every fragment read of the stage goes out before the matrix work
      // (measured: 2-8% faster products than reads interleaved with it)
      __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
      mma(f);
      __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
      if constexpr (SW) asm volatile("" : "+v"(ssq_acc));  // read and added before the next barrier releases the slot
    }
  }
  wait_vm<0>();  // no load may still write this workgroup's LDS
  raw_barrier();

  // ---- epilogue.  lane holds Y[m = (lane & 15) + row base][n = 4*(lane >> 4) + i + column base]
  if constexpr (OUT == OUT_PARTIAL) {
    const int ntiles = g.N >> 4;
#pragma unroll
    for (int fn = 0; fn < NF; ++fn) {
      const int n = n0 + 16 * NF * wn + 16 * fn;
      if (n >= g.N) continue;
#pragma unroll
      for (int fm = 0; fm < MF; ++fm) {
        const int m = m0 + 16 * MF * wm + 16 * fm + (lane & 15);
        if (m < g.M)
          *reinterpret_cast<f32x4*>(g.part + (((size_t)ks * ntiles + (n >> 4)) * g.M + m) * 16 + 4 * (lane >> 4)) =
              acc[fn][fm];
      }
    }
    if (g.rinv_out != nullptr && ks == 0) write_rinv(g, nb * g.nbm + mb, g.nbn * g.nbm);
  } else if constexpr (SW) {
    // the up accumulators (waves wn = 1) meet the gate ones (wn = 0) of the
    // same (row, column) through the idle ring; the rows' scales from the two
    // halves' sums, in a fixed order
    float* sx = reinterpret_cast<float*>(lds);
    float* sh = sx + 4 * NF * MF * 256;  // [512] the halves' sums of squares
    float* rs = sh + 512;                // [256] row scales
    sh[tid] = ssq_acc;
    if (wn == 1) {
#pragma unroll
      for (int fn = 0; fn < NF; ++fn)
#pragma unroll
        for (int fm = 0; fm < MF; ++fm)
          *reinterpret_cast<f32x4*>(sx + (((wm * NF + fn) * MF + fm) * 64 + lane) * 4) = acc[fn][fm];
    }
    __syncthreads();
    if (tid < 256) rs[tid] = 1.0f / sqrtf((sh[tid] + sh[tid + 256]) / (float)g.K + g.eps);
    __syncthreads();
    if (wn == 0) {
      bf16_t* out = reinterpret_cast<bf16_t*>(g.act_out);
#pragma unroll
      for (int fm = 0; fm < MF; ++fm) {
        const int row = 16 * MF * wm + 16 * fm + (lane & 15), m = m0 + row;
        const float r = rs[row];
        if (m >= g.M) continue;
#pragma unroll
        for (int fn = 0; fn < NF; ++fn) {
          const f32x4 u = *reinterpret_cast<const f32x4*>(sx + (((wm * NF + fn) * MF + fm) * 64 + lane) * 4);
          uint32_t w[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t b0 = f32_to_bf16_bits(silu_f32(acc[fn][fm][2 * h] * r) * (u[2 * h] * r));
            const uint32_t b1 = f32_to_bf16_bits(silu_f32(acc[fn][fm][2 * h + 1] * r) * (u[2 * h + 1] * r));
            w[h] = b0 | b1 << 16;
          }
          const int c = 16 * (nb * NF + fn) + 4 * (lane >> 4);
          *reinterpret_cast<u32x2*>(out + (size_t)m * g.ld_act + c) = u32x2{w[0], w[1]};
        }
      }
    }
  } else {
    uint64_t* sb = reinterpret_cast<uint64_t*>(lds);  // [2][BM]; the ring is idle after the last barrier
#pragma unroll
    for (int fm = 0; fm < MF; ++fm) {
      uint64_t best = 0;
#pragma unroll
      for (int fn = 0; fn < NF; ++fn) {
        const int n = n0 + 16 * NF * wn + 16 * fn;
        if (n < g.N) {
          const uint64_t t = tile_row_best(acc[fn][fm], n, lane);
          best = t > best ? t : best;
        }
      }
      if ((lane >> 4) == 0) sb[wn * BM + 16 * MF * wm + 16 * fm + (lane & 15)] = best;
    }
    if (g.logits_dbg != nullptr) {
#pragma unroll
      for (int fn = 0; fn < NF; ++fn) {
        const int n = n0 + 16 * NF * wn + 16 * fn;
        if (n >= g.N) continue;
#pragma unroll
        for (int fm = 0; fm < MF; ++fm) {
          const int m = m0 + 16 * MF * wm + 16 * fm + (lane & 15);
          if (m >= g.M) continue;
          const float r = row_rinv(g.ssq_in, g.ssq_nparts, g.ld_ssq, m, g.K, g.eps);
#pragma unroll
          for (int i = 0; i < 4; ++i) g.logits_dbg[(size_t)m * g.N + n + 4 * (lane >> 4) + i] = acc[fn][fm][i] * r;
        }
      }
    }
    __syncthreads();
    for (int rr = tid; rr < BM; rr += 512) {
      const uint64_t a = sb[rr], b = sb[BM + rr];
      if (m0 + rr < g.M) g.best_part[(size_t)nb * g.ld_best + m0 + rr] = a > b ? a : b;
    }
  }
}

// ------------------------------------------------------------------ argmax reduce
// draft id of each row = index of the largest packed key over the LM-head
// workgroups' keys part[t][m] (t < ntiles, leading dimension ld).  A
// workgroup of 1024 threads covers 16 rows: thread (c, r) = (tid >> 4,
// tid & 15) reads keys t = c, c + 64, ... of row r (16 rows = one contiguous
// 128-byte line per t), 8 loads issued together, then an LDS fold over c.
__global__ void __launch_bounds__(1024) argmax_reduce_kernel(const uint64_t* part, int ntiles, int ld, int M,
                                                             int32_t* ids) {
  __shared__ uint64_t s_best[64][16];
  const int r = threadIdx.x & 15, c = threadIdx.x >> 4;
  const int m = blockIdx.x * 16 + r;
  const bool ok = m < M;
  uint64_t best = 0;
  for (int t0 = c; t0 < ntiles; t0 += 8 * 64) {
    uint64_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = t0 + 64 * i;
      v[i] = ok && t < ntiles ? part[(size_t)t * ld + m] : 0ull;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) best = v[i] > best ? v[i] : best;
  }
  s_best[c][r] = best;
  __syncthreads();
  for (int s = 32; s >= 1; s >>= 1) {
    if (c < s) s_best[c][r] = s_best[c + s][r] > s_best[c][r] ? s_best[c + s][r] : s_best[c][r];
    __syncthreads();
  }
  if (c == 0 && ok) ids[m] = argmax_key_index(s_best[0][r]);
}

// ------------------------------------------------------------------ finish kernels
// Every finish kernel is elementwise over its outputs: a thread takes 4
// consecutive columns of one row (16-byte partial loads) and issues all the
// global loads those outputs need at once (one round of memory latency): the
// k-slice partials, the row scale and the epilogue operands.

// k-slice sums of NQ column quads of one row.  Lane j of the SPL lanes that
// share the quads (KS a multiple of SPL) takes slices j, j + SPL, ... in that
// order, two per round: a round issues both slices' loads unconditionally,
// the index clamped to a valid slice and a surplus value dropped on the ALU
// side.  (Loads behind branches make the compiler copy each result at the
// merge, waiting for it there, and lose the count of loads in flight, so a
// later dependent load would wait for all of them.)
template <int SPL, int NQ>
struct KSlices {
  const float* p[NQ];
  size_t stride;
  int KS;
  f32x4 t[NQ][2];

  __device__ __forceinline__ KSlices(const FinishArgs& f, int m, const int (&n)[NQ], int j) {
    stride = (size_t)f.ntiles * f.M * 16;
    KS = f.KS;
#pragma unroll
    for (int q = 0; q < NQ; ++q) p[q] = f.part + ((size_t)(n[q] >> 4) * f.M + m) * 16 + (n[q] & 15) + j * stride;
  }
  __device__ __forceinline__ void issue(int s0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const size_t sl = (size_t)min(s0 + SPL * i, KS - SPL);
#pragma unroll
      for (int q = 0; q < NQ; ++q) t[q][i] = *reinterpret_cast<const f32x4*>(p[q] + sl * stride);
    }
  }
  __device__ __forceinline__ void add(int s0, f32x4 (&v)[NQ]) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bool in = s0 + SPL * i < KS;
#pragma unroll
      for (int q = 0; q < NQ; ++q) v[q] += in ? t[q][i] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // every round after the first (issued and added by the caller)
  __device__ __forceinline__ void rest(f32x4 (&v)[NQ]) {
    for (int s0 = 2 * SPL; s0 < KS; s0 += 2 * SPL) {
      issue(s0);
      add(s0, v);
    }
  }
};

template <int SPL, int NQ>
__device__ __forceinline__ void ksum(const FinishArgs& f, int m, const int (&n)[NQ], int j, f32x4 (&v)[NQ]) {
  KSlices<SPL, NQ> k(f, m, n, j);
#pragma unroll
  for (int q = 0; q < NQ; ++q) v[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  k.issue(0);
  k.add(0, v);
  k.rest(v);
}

// Sum over the SPL adjacent lanes that share a quad (every lane gets it).
template <int SPL>
__device__ __forceinline__ void group_sum(f32x4& v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (SPL >= 2) v[e] += quad_xor1(v[e]);
    if constexpr (SPL >= 4) v[e] += quad_xor2(v[e]);
  }
}

__device__ __forceinline__ float row_scale(const FinishArgs& f, int m) { return f.rinv != nullptr ? f.rinv[m] : 1.0f; }

// E (1, 2 or 4) consecutive bf16 values packed into one 2-, 4- or 8-byte store.
template <int E>
__device__ __forceinline__ void store_bits(bf16_t* dst, const bf16_t (&b)[E]) {
  if constexpr (E == 4) {
    *reinterpret_cast<u32x2*>(dst) =
        u32x2{(uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16)};
  } else if constexpr (E == 2) {
    *reinterpret_cast<uint32_t*>(dst) = (uint32_t)b[0] | ((uint32_t)b[1] << 16);
  } else {
    *dst = b[0];
  }
}

// E values as a bf16 hi/lo pair at idx (a multiple of E).
template <int E>
__device__ __forceinline__ void split_store(bf16_t* hi, bf16_t* lo, size_t idx, const float (&v)[E]) {
  bf16_t h[E], l[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    h[e] = f32_to_bf16_bits(v[e]);
    l[e] = f32_to_bf16_bits(v[e] - bf16_bits_to_f32(h[e]));
  }
  store_bits<E>(hi + idx, h);
  if (lo) store_bits<E>(lo + idx, l);
}

// E values in the storage type at dst (aligned to E elements).
template <typename S, int E>
__device__ __forceinline__ void store_n(S* dst, const float (&v)[E]) {
  if constexpr (sizeof(S) == 4) {
    if constexpr (E == 4) *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
    else if constexpr (E == 2) *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
    else *dst = v[0];
  } else {
    bf16_t b[E];
#pragma unroll
    for (int e = 0; e < E; ++e) b[e] = f32_to_bf16_bits(v[e]);
    store_bits<E>(dst, b);
  }
}

// E consecutive floats from src (aligned to E elements).
template <int E>
__device__ __forceinline__ void load_n(const float* src, float (&v)[E]) {
  if constexpr (E == 4) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = t[e];
  } else if constexpr (E == 2) {
    const float2 t = *reinterpret_cast<const float2*>(src);
    v[0] = t.x;
    v[1] = t.y;
  } else {
    v[0] = *src;
  }
}

// Elements j*E .. j*E + E-1 of a quad (lane j of the SPL = 4/E lanes sharing
// it), picked by selects rather than a dynamic register index.
template <int E>
__device__ __forceinline__ void pick(const f32x4& v, int j, float (&o)[E]) {
  if constexpr (E == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = v[e];
  } else if constexpr (E == 2) {
    o[0] = j ? v[2] : v[0];
    o[1] = j ? v[3] : v[1];
  } else {
    o[0] = j == 0 ? v[0] : (j == 1 ? v[1] : (j == 2 ? v[2] : v[3]));
  }
}

// 8-bit cache entries of this lane: E values at column c (lo) and c + half
// (hi) of a cache row.  The 8 * SPL consecutive lanes holding 4 consecutive
// rotation pairs each cover one run of 32 values in each half (the runs of a
// head row are dims [0, 32), [32, 64), ...; D is 64 or 128, so a half holds
// whole runs), and share its scale s = max|x| / 127; the values are
// q = x / s rounded half to even (0 for a run of zeros).  The first lane of
// the run writes its scale.
template <int SPL, int E>
__device__ __forceinline__ void store_kv8(int8_t* vals, float* scales, size_t c, int half, const float (&lo)[E],
                                          const float (&hi)[E]) {
  constexpr int RUN = 8 * SPL;  // lanes per run
  float alo = 0.f, ahi = 0.f;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    alo = fmaxf(alo, fabsf(lo[k]));
    ahi = fmaxf(ahi, fabsf(hi[k]));
  }
#pragma unroll
  for (int o = 1; o < RUN; o <<= 1) {
    alo = fmaxf(alo, __shfl_xor(alo, o));
    ahi = fmaxf(ahi, __shfl_xor(ahi, o));
  }
  const float slo = alo / 127.0f, shi = ahi / 127.0f;
  auto pack = [&](const float (&v)[E], float sc, int8_t* dst) {
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < E; ++k) {
      const float q = sc > 0.f ? fminf(fmaxf(rintf(v[k] / sc), -127.f), 127.f) : 0.f;
      w |= ((uint32_t)(int32_t)q & 0xffu) << (8 * k);
    }
    if constexpr (E == 4) *reinterpret_cast<uint32_t*>(dst) = w;
    else if constexpr (E == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w;
    else *dst = (int8_t)w;
  };
  pack(lo, slo, vals + c);
  pack(hi, shi, vals + c + half);
  if ((threadIdx.x & (RUN - 1)) == 0) {
    scales[c >> 5] = slo;
    scales[(c + half) >> 5] = shi;
  }
}

// Rotation of the pair (lo, hi) by the tabulated angle of (position, pair index).
__device__ __forceinline__ void rope_apply(float& lo, float& hi, float2 cs) {
  const float a = lo, b = hi;
  lo = a * cs.x - b * cs.y;
  hi = a * cs.y + b * cs.x;
}

// The E tabulated (cos, sin) of pairs d .. d + E-1 at position pos (d a
// multiple of E).
template <int E>
__device__ __forceinline__ void rope_n(const FinishArgs& f, int pos, int d, float2 (&cs)[E]) {
  const float2* t = f.rope + (size_t)pos * (f.head_dim >> 1) + d;
  if constexpr (E == 1) {
    cs[0] = t[0];
  } else {
#pragma unroll
    for (int h = 0; h < E / 2; ++h) {
      const f32x4 a = reinterpret_cast<const f32x4*>(t)[h];
      cs[2 * h] = make_float2(a[0], a[1]);
      cs[2 * h + 1] = make_float2(a[2], a[3]);
    }
  }
}

// y = sum (+ x residual, + width-3 block conv); x / out_f32 = y; hi/lo of
// y * gnext (row-major, or in fragment blocks for an LDS-DMA consumer); sums
// of squares per (tile, row).  grid: (tiles / (4/SPL), row
// groups of 16); thread t: lane j = t % SPL of the group sharing column quad
// q = (t / SPL) & 3 of row r = (t / 4SPL) & 15 of tile t / 64SPL, each lane
// finishing 4/SPL columns.  The conv's neighbour rows come through LDS (a
// conv block never crosses a 16-row group: the block divides 16).
template <typename S, int SPL>
__global__ void __launch_bounds__(256) finish_rowtile_kernel(const FinishArgs f) {
  constexpr int E = 4 / SPL, TPB = 4 / SPL;  // columns per lane, tiles per workgroup
  __shared__ float s_y[TPB][16][16];
  const int t = threadIdx.x, j = t % SPL, q = (t / SPL) & 3, r = (t / (4 * SPL)) & 15, tl = t / (64 * SPL);
  const int tile = blockIdx.x * TPB + tl;
  const int m = 16 * blockIdx.y + r, n = tile * 16 + 4 * q, col = 4 * q + j * E;
  const bool ok = m < f.M && tile < f.ntiles;
  const size_t idx = (size_t)m * f.N + n + j * E;
  // epilogue operands of this lane's columns first: their loads fly with the partial loads
  float xr[E], gn[E], c0[E], c1[E], c2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) xr[e] = gn[e] = c0[e] = c1[e] = c2[e] = 0.f;
  if (ok) {
    if (f.x != nullptr) load_n<E>(f.x + idx, xr);
    const S* g = reinterpret_cast<const S*>(f.gnext) + n + j * E;
#pragma unroll
    for (int e = 0; e < E; ++e) gn[e] = load_f32<S>(g + e);
    if (f.conv != nullptr) {
      const S* cw = reinterpret_cast<const S*>(f.conv) + 3 * (n + j * E);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        c0[e] = load_f32<S>(cw + 3 * e);
        c1[e] = load_f32<S>(cw + 3 * e + 1);
        c2[e] = load_f32<S>(cw + 3 * e + 2);
      }
    }
  }
  // (unconditional loads: a row past M reads row M - 1 and drops it; the grid covers the tiles exactly)
  f32x4 v4[1];
  ksum<SPL, 1>(f, min(m, f.M - 1), {n}, j, v4);
  if (!ok) v4[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  group_sum<SPL>(v4[0]);
  float v[E], y[E];
  pick<E>(v4[0], j, v);
#pragma unroll
  for (int e = 0; e < E; ++e) y[e] = v[e] = v[e] + xr[e];
  if (f.conv != nullptr) {
#pragma unroll
    for (int e = 0; e < E; ++e) s_y[tl][r][col + e] = v[e];
    __syncthreads();
    const int i = m % f.block;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float c = c1[e] * v[e];
      if (i > 0) c += c0[e] * s_y[tl][r - 1][col + e];
      if (i < f.block - 1 && m + 1 < f.M) c += c2[e] * s_y[tl][r + 1][col + e];
      y[e] = v[e] + c;
    }
  }
  float sq = 0.f;
  if (ok) {
    if (f.x != nullptr) store_n<float, E>(f.x + idx, y);
    if (f.out_f32 != nullptr) store_n<float, E>(f.out_f32 + idx, y);
    float sv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      sv[e] = y[e] * gn[e];
      sq += y[e] * y[e];
    }
    // (fragment blocks: the lane's E columns stay inside one 8-column piece)
    const size_t oidx = f.out_blocked ? frag_block_index(m, n + j * E, f.N) : idx;
    split_store<E>(reinterpret_cast<bf16_t*>(f.out_hi), reinterpret_cast<bf16_t*>(f.out_lo), oidx, sv);
  }
  // the row's 4 SPL lanes
  sq += quad_xor1(sq);
  sq += quad_xor2(sq);
#pragma unroll
  for (int o = 4; o < 4 * SPL; o <<= 1) sq += __shfl_xor(sq, o);
  if (q == 0 && j == 0 && ok) f.ssq_out[(size_t)tile * f.ld_ssq + m] = sq;
}

// act[m, c] = silu(rinv * y_gate) * (rinv * y_up) as a hi/lo pair.  SPL
// lanes per 4 outputs, ordered (tile, row, quad) so the partial reads are
// contiguous; after the lanes' sums are combined each finishes 4/SPL outputs.
template <int SPL>
__global__ void __launch_bounds__(256) finish_swiglu_kernel(const FinishArgs f) {
  constexpr int E = 4 / SPL;
  const int F = f.N >> 1;
  const int e = blockIdx.x * blockDim.x + threadIdx.x, e4 = e / SPL, j = e % SPL;
  if (e4 >= f.M * (F >> 2)) return;  // whole lane groups leave together
  const int tile = e4 / (f.M * 4), rem = e4 - tile * (f.M * 4);
  const int m = rem >> 2, c = tile * 16 + 4 * (rem & 3);
  const float r = row_scale(f, m);
  f32x4 gu[2];
  ksum<SPL, 2>(f, m, {c, F + c}, j, gu);
  group_sum<SPL>(gu[0]);
  group_sum<SPL>(gu[1]);
  float g[E], u[E], a[E];
  pick<E>(gu[0], j, g);
  pick<E>(gu[1], j, u);
#pragma unroll
  for (int k = 0; k < E; ++k) a[k] = silu_f32(g[k] * r) * (u[k] * r);
  split_store<E>(reinterpret_cast<bf16_t*>(f.out_hi), reinterpret_cast<bf16_t*>(f.out_lo), (size_t)m * F + c + j * E,
                 a);
}

// Block Q/K/V: RoPE on Q and K at position T + i (T = ctx_len[b], clamped);
// Q scaled and stored as a hi/lo pair; K and V staged in this layer's cache at
// rows T + i (rows past the committed context: the attention reads every key
// from the cache).  A sequence whose block would pass max_ctx stages nothing
// and is flagged.  SPL lanes per 4 consecutive rotation pairs (row, head of
// the concatenated [Q | K | V] output, d .. d + 3 < D/2); each lane finishes
// 4/SPL of them.
template <typename S, int SPL, bool KV8>
__global__ void __launch_bounds__(256) finish_qkv_kernel(const FinishArgs f) {
  constexpr int E = 4 / SPL;
  const int D = f.head_dim, half = D >> 1;
  const int quads = f.N >> 3;  // 4-pair groups per row
  const int e = blockIdx.x * blockDim.x + threadIdx.x, e4 = e / SPL, j = e % SPL;
  if (e4 >= f.M * quads) return;  // whole lane groups leave together
  int m, hd, d;
  if (KV8 || f.M < 256) {
    // (row, head, pair): the lanes of one run of 32 values of a head row are
    // consecutive (the 8-bit cache's run maximum is a shuffle reduction), and
    // a row's stores are contiguous
    m = e4 / quads;
    const int rem = e4 - m * quads;
    hd = rem / (half >> 2);
    d = (rem - hd * (half >> 2)) * 4;
  } else {
    // from 256 rows on, where the partials dominate the traffic: (head,
    // 16-pair group, row, quad), so 4 lanes read a row's 64 contiguous bytes
    // of a partial tile and the lanes of 16 rows its whole 1 KB (batch 32:
    // 89 -> 83 us per Q/K/V stage)
    const int q = e4 & 3, r2 = e4 >> 2, pidx = r2 / f.M;
    m = r2 - pidx * f.M;
    hd = pidx / (half >> 4);
    d = (pidx - hd * (half >> 4)) * 16 + 4 * q;
  }
  const int n = hd * D + d, nj = n + j * E;  // nj: this lane's first pair
  const int Nq = f.n_q_heads * D, Nk = f.n_kv_heads * D;
  const int b = m / f.block, i = m - b * f.block;
  const float r = row_scale(f, m);
  // a caller-set length outside [0, max_ctx] is clamped (the table covers every clamped position)
  const int T = min(max(f.ctx_len[b], 0), f.max_ctx);
  const int pos = T + i;
  // the first round of partial loads goes out before the table load that
  // waits for the context length
  KSlices<SPL, 2> ks(f, m, {n, n + half}, j);
  ks.issue(0);
  float2 cs[E];
  rope_n<E>(f, pos, d + j * E, cs);
  f32x4 v[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  ks.add(0, v);
  ks.rest(v);
  group_sum<SPL>(v[0]);
  group_sum<SPL>(v[1]);
  float lo[E], hi[E];
  pick<E>(v[0], j, lo);
  pick<E>(v[1], j, hi);
#pragma unroll
  for (int k = 0; k < E; ++k) {
    lo[k] *= r;
    hi[k] *= r;
  }
  if (n < Nq) {
    bf16_t* qh = reinterpret_cast<bf16_t*>(f.out_hi);
    bf16_t* ql = reinterpret_cast<bf16_t*>(f.out_lo);
#pragma unroll
    for (int k = 0; k < E; ++k) {
      rope_apply(lo[k], hi[k], cs[k]);
      lo[k] *= f.q_scale;
      hi[k] *= f.q_scale;
    }
    split_store<E>(qh, ql, (size_t)m * Nq + nj, lo);
    split_store<E>(qh, ql, (size_t)m * Nq + nj + half, hi);
    return;
  }
  if (T + f.block > f.max_ctx) {
    if (n == Nq && i == 0 && j == 0) atomicOr(f.err, kErrDraftOverflow);
    return;
  }
  const bool is_k = n < Nq + Nk;
  const int c = (is_k ? n - Nq : n - Nq - Nk) + j * E;  // column within the KV heads
  if (is_k) {
#pragma unroll
    for (int k = 0; k < E; ++k) rope_apply(lo[k], hi[k], cs[k]);
  }
  const size_t at = ((size_t)b * f.max_ctx + pos) * Nk + c;
  if constexpr (KV8) {
    store_kv8<SPL, E>(reinterpret_cast<int8_t*>(f.kv_cache[is_k ? 0 : 1]), f.kv_scale[is_k ? 0 : 1], at, half, lo, hi);
  } else {
    S* dst = reinterpret_cast<S*>(f.kv_cache[is_k ? 0 : 1]) + at;
    store_n<S, E>(dst, lo);
    store_n<S, E>(dst + half, hi);
  }
}

// Context K/V of every layer (segments K^0, V^0, K^1, V^1, ...): RoPE on K at
// position ctx_len[b] + i, scatter to cache row ctx_len[b] + i.  A sequence
// whose rows would pass max_ctx is skipped and flagged.  SPL lanes per 4
// consecutive rotation pairs (row, head of the concatenated output, d .. d+3);
// each lane finishes 4/SPL of them.
template <typename S, int SPL, bool KV8>
__global__ void __launch_bounds__(256) finish_kv_kernel(const FinishArgs f) {
  constexpr int E = 4 / SPL;
  const int D = f.head_dim, half = D >> 1, Hkv = f.n_kv_heads;
  const int quads = f.N >> 3;
  const int e = blockIdx.x * blockDim.x + threadIdx.x, e4 = e / SPL, j = e % SPL;
  if (e4 >= f.M * quads) return;  // whole lane groups leave together
  int m, hd, d;
  if (KV8 || f.M < 256) {  // lane order as in finish_qkv
    m = e4 / quads;
    const int rem = e4 - m * quads;
    hd = rem / (half >> 2);
    d = (rem - hd * (half >> 2)) * 4;
  } else {
    const int q = e4 & 3, r2 = e4 >> 2, pidx = r2 / f.M;
    m = r2 - pidx * f.M;
    hd = pidx / (half >> 4);
    d = (pidx - hd * (half >> 4)) * 16 + 4 * q;
  }
  const int seg = hd / Hkv, head = hd - seg * Hkv;
  const int b = m / f.block, i = m - b * f.block;
  const int n = hd * D + d;
  const float r = row_scale(f, m);
  const int t0 = f.ctx_len[b];
  const bool bad = t0 < 0 || t0 + f.block > f.max_ctx;
  const int pos = bad ? 0 : t0 + i;
  KSlices<SPL, 2> ks(f, m, {n, n + half}, j);
  ks.issue(0);
  float2 cs[E];
#pragma unroll
  for (int k = 0; k < E; ++k) cs[k] = make_float2(1.f, 0.f);
  if ((seg & 1) == 0) rope_n<E>(f, pos, d + j * E, cs);
  f32x4 v[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  ks.add(0, v);
  ks.rest(v);
  group_sum<SPL>(v[0]);
  group_sum<SPL>(v[1]);
  if (bad) {
    if (n == 0 && i == 0 && j == 0) atomicOr(f.err, kErrFuseOverflow);
    return;
  }
  float lo[E], hi[E];
  pick<E>(v[0], j, lo);
  pick<E>(v[1], j, hi);
#pragma unroll
  for (int k = 0; k < E; ++k) {
    lo[k] *= r;
    hi[k] *= r;
    if ((seg & 1) == 0) rope_apply(lo[k], hi[k], cs[k]);
  }
  const size_t at = (((size_t)b * f.max_ctx + pos) * Hkv + head) * D + d + j * E;
  if constexpr (KV8) {
    store_kv8<SPL, E>(reinterpret_cast<int8_t*>(f.kv_cache[seg]), f.kv_scale[seg], at, half, lo, hi);
  } else {
    S* dst = reinterpret_cast<S*>(f.kv_cache[seg]) + at;
    store_n<S, E>(dst, lo);
    store_n<S, E>(dst + half, hi);
  }
}

// ------------------------------------------------------------------ weight tiling
// One 16-byte fragment per thread: fragment p is lane p & 63 of block
// p >> 6 = (tile t, k-step s).  Streaming a k-step of a tile is then one
// contiguous 1 KB read instead of 16 rows x 64 B: a probe streaming the
// LM-head matrix measured 7.0 TB/s against 6.1 TB/s, the flat-read ceiling
// of the box being 7.1 TB/s.
template <typename S>
__global__ void tile_weights_kernel(const S* src, int rows, int K, bf16_t* dst, int tile0) {
  const int nks = K >> 5;
  const size_t n = (size_t)(rows >> 4) * nks * 64;
  for (size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x; p < n; p += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(p & 63);
    const size_t b = p >> 6;
    const int t = (int)(b / nks), s = (int)(b - (size_t)t * nks);
    Raw8 r;
    load_raw8<S>(r, src + (size_t)(16 * t + (l & 15)) * K + 32 * s + 8 * (l >> 4));
    *reinterpret_cast<bf16x8*>(dst + (((size_t)(tile0 + t) * nks + s) * 64 + l) * 8) = raw_to_bf16x8<S>(r);
  }
}

hipError_t launch_tile_weights(int storage, const void* src, int rows, int K, void* dst, int tile0,
                               hipStream_t stream) {
  const size_t n = (size_t)(rows / 16) * (K / 32) * 64;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 8192);
  if (storage == ST_BF16)
    hipLaunchKernelGGL(tile_weights_kernel<bf16_t>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(src), rows, K, static_cast<bf16_t*>(dst), tile0);
  else
    hipLaunchKernelGGL(tile_weights_kernel<float>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const float*>(src), rows, K, static_cast<bf16_t*>(dst), tile0);
  return hipGetLastError();
}

// ------------------------------------------------------------------ launchers
int gemm_as_ksl(int M, int K, bool lo, bool argmax, int ntiles, int cus) {
  const int MR = M <= 16 ? 1 : (M <= 32 ? 2 : 0);
  if (MR == 0) return 0;
  const int narr = lo ? 2 : 1;
  const int step = 256;  // whole register stages at either MR
  auto lds = [&](int ksl) { return (size_t)narr * 16 * MR * (ksl + 8) * 2; };
  if (K % step) return 0;
  if (argmax) return lds(K) <= kGemmAsMaxLds ? K : 0;
  // the longest slice (fewest partials) that still gives every compute unit
  // 8 tile-slices to stream, else the shortest slice that fits
  int best = 0;
  for (int ksl = step; ksl <= K; ksl += step) {
    if (K % ksl || lds(ksl) > kGemmAsSliceLds) continue;
    if (best == 0 || (long)ntiles * (K / ksl) >= 8L * cus) best = ksl;
  }
  return best;
}

size_t gemm_as_lds(int M, int ksl, bool lo) {
  const int MR = M <= 16 ? 1 : 2;
  return (size_t)(lo ? 2 : 1) * 16 * MR * (ksl + 8) * 2;
}


template <typename Kern>
static void allow_lds(Kern kernel, size_t bytes) {
  (void)allow_dynamic_lds(reinterpret_cast<const void*>(kernel), bytes);
}

template <typename S, int MR, int SRC, bool LO, int OUT>
static hipError_t launch_as(const GemmArgs& a, const GemmLaunch& l, hipStream_t st) {
  auto k = gemm_as_kernel<S, MR, SRC, LO, OUT>;
  allow_lds(k, l.lds);
  hipLaunchKernelGGL(k, l.grid, dim3(l.threads), l.lds, st, a);
  return hipGetLastError();
}
template <typename S, int MF, int NF, int SRC, bool LO, int OUT>
static hipError_t launch_mt(const GemmArgs& a, const GemmLaunch& l, hipStream_t st) {
  auto k = gemm_mt_kernel<S, MF, NF, SRC, LO, OUT>;
  allow_lds(k, l.lds);
  hipLaunchKernelGGL(k, l.grid, dim3(l.threads), l.lds, st, a);
  return hipGetLastError();
}

template <int MF, int NF, int SRC, bool LO, int OUT>
static hipError_t launch_dma(const GemmArgs& a, const GemmLaunch& l, hipStream_t st) {
  auto k = gemm_dma_kernel<MF, NF, SRC, LO, OUT>;
  allow_lds(k, l.lds);
  hipLaunchKernelGGL(k, l.grid, dim3(l.threads), l.lds, st, a);
  return hipGetLastError();
}

template <typename S, int SRC, bool LO, int OUT>
static hipError_t dispatch_mr(const GemmArgs& a, const GemmLaunch& l, hipStream_t st) {
  if (l.kind == GEMM_DMA) {
    if constexpr (sizeof(S) == 2) {
      if (l.MR == 4) {
        if (l.NF == 8) return launch_dma<4, 8, SRC, LO, OUT>(a, l, st);
        if constexpr (OUT == OUT_PARTIAL)
          if (l.NF == 6) return launch_dma<4, 6, SRC, LO, OUT>(a, l, st);
      } else if (l.MR <= 2) {
        // (the fusion at 64 and 128 rows)
        if constexpr (SRC == SRC_CONCAT && OUT == OUT_PARTIAL) {
          if (l.MR == 1) {
            switch (l.NF) {
              case 2: return launch_dma<1, 2, SRC, LO, OUT>(a, l, st);
              case 4: return launch_dma<1, 4, SRC, LO, OUT>(a, l, st);
              case 6: return launch_dma<1, 6, SRC, LO, OUT>(a, l, st);
              case 8: return launch_dma<1, 8, SRC, LO, OUT>(a, l, st);
            }
          } else {
            switch (l.NF) {
              case 2: return launch_dma<2, 2, SRC, LO, OUT>(a, l, st);
              case 4: return launch_dma<2, 4, SRC, LO, OUT>(a, l, st);
              case 5: return launch_dma<2, 5, SRC, LO, OUT>(a, l, st);
              case 6: return launch_dma<2, 6, SRC, LO, OUT>(a, l, st);
            }
          }
        }
      } else if (l.MR == 3) {
        if (l.NF == 8) return launch_dma<3, 8, SRC, LO, OUT>(a, l, st);
        if constexpr (OUT == OUT_PARTIAL)
          if (l.NF == 6) return launch_dma<3, 6, SRC, LO, OUT>(a, l, st);
      }
    }
    return hipErrorInvalidValue;
  }
  if (l.kind == GEMM_AS) {
    if (l.MR == 1) return launch_as<S, 1, SRC, LO, OUT>(a, l, st);
    if (l.MR == 2) return launch_as<S, 2, SRC, LO, OUT>(a, l, st);
    return hipErrorInvalidValue;
  }
  switch (l.MR) {  // GEMM_MT: MR = MF
    case 1:
      switch (l.NF) {
        case 2: return launch_mt<S, 1, 2, SRC, LO, OUT>(a, l, st);
        case 4: return launch_mt<S, 1, 4, SRC, LO, OUT>(a, l, st);
        case 6: return launch_mt<S, 1, 6, SRC, LO, OUT>(a, l, st);
        case 8: return launch_mt<S, 1, 8, SRC, LO, OUT>(a, l, st);
      }
      return hipErrorInvalidValue;
    case 2:
      switch (l.NF) {
        case 2: return launch_mt<S, 2, 2, SRC, LO, OUT>(a, l, st);
        case 4: return launch_mt<S, 2, 4, SRC, LO, OUT>(a, l, st);
        case 5: return launch_mt<S, 2, 5, SRC, LO, OUT>(a, l, st);
        case 6: return launch_mt<S, 2, 6, SRC, LO, OUT>(a, l, st);
      }
      return hipErrorInvalidValue;
    case 4:
      if constexpr (OUT == OUT_PARTIAL)
        if (l.NF == 6) return launch_mt<S, 4, 6, SRC, LO, OUT>(a, l, st);
      return launch_mt<S, 4, 8, SRC, LO, OUT>(a, l, st);
  }
  return hipErrorInvalidValue;
}

template <typename S>
static hipError_t dispatch_s(const GemmArgs& a, const GemmLaunch& l, hipStream_t st) {
  if (l.out == OUT_SWIGLU) {
    if constexpr (sizeof(S) == 2)
      if (l.kind == GEMM_DMA && l.src == SRC_SPLIT && !l.lo && l.MR == 4 && l.NF == 6 && l.KS == 1 &&
          a.ssq_nparts == a.K / 16 && a.kslice == a.K && a.N % 192 == 0)
        return launch_dma<4, 6, SRC_SPLIT, false, OUT_SWIGLU>(a, l, st);
    return hipErrorInvalidValue;
  }
  if (l.src == SRC_CONCAT) {
    if (l.out != OUT_PARTIAL) return hipErrorInvalidValue;
    // fp32 sources are split on the fly; bf16 sources are exact
    if constexpr (sizeof(S) == 4) return dispatch_mr<S, SRC_CONCAT, true, OUT_PARTIAL>(a, l, st);
    else return dispatch_mr<S, SRC_CONCAT, false, OUT_PARTIAL>(a, l, st);
  }
  if (l.out == OUT_ARGMAX)
    return l.lo ? dispatch_mr<S, SRC_SPLIT, true, OUT_ARGMAX>(a, l, st)
                : dispatch_mr<S, SRC_SPLIT, false, OUT_ARGMAX>(a, l, st);
  return l.lo ? dispatch_mr<S, SRC_SPLIT, true, OUT_PARTIAL>(a, l, st)
              : dispatch_mr<S, SRC_SPLIT, false, OUT_PARTIAL>(a, l, st);
}

hipError_t launch_gemm(int storage, const GemmArgs& a, const GemmLaunch& l, hipStream_t stream) {
  // only the LDS-DMA kernel reads activations stored in fragment blocks
  if (a.a_blocked && (l.kind != GEMM_DMA || l.src != SRC_SPLIT || a.K % 32)) return hipErrorInvalidValue;
  if (storage == ST_BF16) return dispatch_s<bf16_t>(a, l, stream);
  return dispatch_s<float>(a, l, stream);
}

hipError_t launch_argmax_reduce(const uint64_t* part, int ntiles, int ld, int M, int32_t* ids, hipStream_t stream) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3((M + 15) / 16), dim3(1024), 0, stream, part, ntiles, ld, M, ids);
  return hipGetLastError();
}

template <typename S, int SPL>
static void launch_finish_spl(FinishKind kind, const FinishArgs& f, int blocks, int threads, hipStream_t st) {
  if (kind == FIN_SWIGLU) {
    hipLaunchKernelGGL(finish_swiglu_kernel<SPL>, dim3(blocks), dim3(threads), 0, st, f);
  } else if (kind == FIN_QKV) {
    if (f.kv_int8) hipLaunchKernelGGL((finish_qkv_kernel<S, SPL, true>), dim3(blocks), dim3(threads), 0, st, f);
    else hipLaunchKernelGGL((finish_qkv_kernel<S, SPL, false>), dim3(blocks), dim3(threads), 0, st, f);
  } else {
    if (f.kv_int8) hipLaunchKernelGGL((finish_kv_kernel<S, SPL, true>), dim3(blocks), dim3(threads), 0, st, f);
    else hipLaunchKernelGGL((finish_kv_kernel<S, SPL, false>), dim3(blocks), dim3(threads), 0, st, f);
  }
}

template <typename S>
static hipError_t launch_finish_s(FinishKind kind, const FinishArgs& f, hipStream_t st) {
  // 4 outputs (FIN_SWIGLU: of N/2 per row) or 4 rotation pairs per lane
  // group; groups of 4 or 2 lanes, splitting the k-slices (KS a multiple of
  // the group), when one lane per quad would leave compute units idle
  const bool few = kind == FIN_ROWTILE ? (size_t)((f.N / 16 + 3) / 4) * ((f.M + 15) / 16) < (size_t)kCUs
                                       : ((size_t)f.M * (f.N / 8) + 255) / 256 < (size_t)kCUs;
  // (a lane takes two slices a round: a group only as wide as keeps both useful)
  int spl = 1;
  if (few) spl = f.KS % 4 == 0 && f.KS >= 8 ? 4 : (f.KS % 2 == 0 && f.KS >= 4 ? 2 : 1);
  if (f.out_blocked && (kind != FIN_ROWTILE || f.N % 32)) return hipErrorInvalidValue;
  if (kind == FIN_ROWTILE) {
    const dim3 grid((f.N / 16 + 4 / spl - 1) / (4 / spl), (f.M + 15) / 16);
    if (spl == 4) hipLaunchKernelGGL((finish_rowtile_kernel<S, 4>), grid, dim3(256), 0, st, f);
    else if (spl == 2) hipLaunchKernelGGL((finish_rowtile_kernel<S, 2>), grid, dim3(256), 0, st, f);
    else hipLaunchKernelGGL((finish_rowtile_kernel<S, 1>), grid, dim3(256), 0, st, f);
    return hipGetLastError();
  }
  if (kind != FIN_SWIGLU && kind != FIN_QKV && kind != FIN_KV) return hipErrorInvalidValue;
  // (a small grid goes out in one-wave workgroups: the dispatcher then spreads
  // the waves evenly over the compute units, whose bandwidth bounds it)
  const size_t quads = (size_t)f.M * (f.N / 8);
  const int threads = few ? 64 : 256;
  const int blocks = (int)((quads * spl + threads - 1) / threads);
  if (spl == 4) launch_finish_spl<S, 4>(kind, f, blocks, threads, st);
  else if (spl == 2) launch_finish_spl<S, 2>(kind, f, blocks, threads, st);
  else launch_finish_spl<S, 1>(kind, f, blocks, threads, st);
  return hipGetLastError();
}

hipError_t launch_finish(int storage, FinishKind kind, const FinishArgs& f, hipStream_t stream) {
  if (storage == ST_BF16) return launch_finish_s<bf16_t>(kind, f, stream);
  return launch_finish_s<float>(kind, f, stream);
}

}  // namespace dfl
