// Weight-streaming matrix-core GEMM for the skinny products of the drafting
// hot path: Y[M, N] = A[M, K] . W[N, K]^T with M = rows of a drafted block
// (or verified rows for the fusion), N, K up to the vocabulary.
//
// Design (gfx950, 64-wide waves):
//  * A workgroup owns NT = 16*WN output columns (weight rows) and MT = 16*MR
//    output rows; its WN x WK waves split the columns 16 rows each (WN) and
//    the reduction dimension (WK).  Each weight element is loaded from HBM
//    exactly once, straight into registers in the 16x16x32 MFMA operand
//    layout (16 rows x 64 contiguous bytes per load instruction, non-temporal
//    so the stream does not evict activations from L2).
//  * Activations arrive as a pair of bf16 arrays (hi, lo) with a = hi + lo,
//    written once by the producing kernel; each fragment costs two MFMAs.
//    The activation then carries about 16 mantissa bits, so only the weights
//    are bf16 -- a plain bf16 activation path loses about 1% of the final
//    hidden state over five random layers.  RMSNorm is applied as a row
//    scale: producers store hi/lo of (x * gain) and the consumer multiplies
//    its result rows by 1/rms computed from the producer's partial sums of
//    squares (the product is linear in the row scale).
//  * Loads for the next unrolled step are issued before the MFMAs of the
//    current one (two register stages).
//  * The WK partial tiles are summed in a fixed order through LDS
//    (deterministic, no float atomics), then a per-tile epilogue runs with
//    the whole MT x NT tile in LDS: this is what lets RoPE pair column d with
//    d + D/2 and SwiGLU pair gate row f with up row f (tile rows come in two
//    halves P rows apart), and the block conv read rows i-1 and i+1.
#include "common.h"
#include "kernels.h"

namespace dfl {

__device__ __forceinline__ int tile_row(int tile, int j, int NT, int P) {
  if (P == 0) return tile * NT + j;
  const int half = NT >> 1;
  const int per = P / half;
  return (tile / per) * 2 * P + (tile % per) * half + (j % half) + (j / half) * P;
}

// Threads per workgroup the register budget allows.
__host__ __device__ constexpr int gemm_max_threads_for(bool wide, int MR) {
  return MR <= 2 ? (wide ? 512 : 1024) : (MR == 4 ? 512 : 256);
}

template <typename S, int MR, int PRO>
struct GemmShape {
  static constexpr int MT = 16 * MR;
  static constexpr int U = MR == 1 ? 4 : (MR == 2 ? 2 : 1);  // k-steps per register stage
  static constexpr bool WIDE = PRO == PRO_SPLIT || sizeof(S) == 4;
  static constexpr int MAXT = gemm_max_threads_for(WIDE, MR);
};

template <typename S, int MR, int PRO>
struct Stage {
  Raw8 w[GemmShape<S, MR, PRO>::U];
  Raw8 a[GemmShape<S, MR, PRO>::U][MR];  // split: .lo = hi bits, .hi = lo bits
};

__device__ __forceinline__ void rope_pair(float& lo, float& hi, int pos, int d, int D, float theta) {
  const double inv_freq = exp(-(2.0 * (double)d / (double)D) * log((double)theta));
  double s, c;
  sincos((double)pos * inv_freq, &s, &c);
  const float cf = (float)c, sf = (float)s;
  const float a = lo, b = hi;
  lo = a * cf - b * sf;
  hi = a * sf + b * cf;
}

// v -> (hi, lo) bf16 pair with v ~= hi + lo.
__device__ __forceinline__ void split_store(bf16_t* hi, bf16_t* lo, size_t idx, float v) {
  const bf16_t h = f32_to_bf16_bits(v);
  hi[idx] = h;
  lo[idx] = f32_to_bf16_bits(v - bf16_bits_to_f32(h));
}

template <typename S, int MR, int PRO, int EPI>
__global__ void __launch_bounds__((GemmShape<S, MR, PRO>::MAXT)) gemm_ws_kernel(const GemmArgs g) {
  constexpr int MT = GemmShape<S, MR, PRO>::MT;
  constexpr int U = GemmShape<S, MR, PRO>::U;
  extern __shared__ __align__(16) float smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x;
  const int WN = g.WN, WK = g.WK;
  const int wn = wave % WN, wk = wave / WN;
  const int NT = 16 * WN;
  const int tile = blockIdx.x;
  const int m0 = blockIdx.y * MT;

  float* red = smem;                    // [WK][MT][NT]
  float* rinv_s = smem + WK * MT * NT;  // [MT]
  float* aux = rinv_s + MT;             // [MT][NT]

  const bool row_scale = PRO == PRO_SPLIT && g.ssq_in != nullptr;

  // ---- the 16 weight rows of this wave
  const int n0 = tile_row(tile, 16 * wn, NT, g.P);
  int sgi = 0;
  while (sgi + 1 < g.nseg && n0 >= g.seg_start[sgi + 1]) ++sgi;
  const S* wp = reinterpret_cast<const S*>(g.seg_ptr[sgi]) +
                (size_t)(n0 - g.seg_start[sgi] + (lane & 15)) * g.K + (size_t)wk * g.kw + (lane >> 4) * 8;

  // ---- activation rows of this lane (padding rows clamp to the last real row)
  int arow[MR];
#pragma unroll
  for (int mi = 0; mi < MR; ++mi) arow[mi] = min(m0 + 16 * mi + (lane & 15), g.M - 1);
  const int kbase = wk * g.kw + (lane >> 4) * 8;

  auto fetch = [&](Stage<S, MR, PRO>& st, int it) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = (it * U + u) * 32;
      load_raw8_nt<S>(st.w[u], wp + ks);
      const int k = kbase + ks;
      if constexpr (PRO == PRO_SPLIT) {
        const bf16_t* ah = reinterpret_cast<const bf16_t*>(g.a_hi);
        const bf16_t* al = reinterpret_cast<const bf16_t*>(g.a_lo);
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) {
          const size_t o = (size_t)arow[mi] * g.lda + k;
          st.a[u][mi].lo = *reinterpret_cast<const u32x4*>(ah + o);
          st.a[u][mi].hi = *reinterpret_cast<const u32x4*>(al + o);
        }
      } else {  // PRO_CONCAT
        const int kstep = wk * g.kw + ks;  // uniform across the wave
        const int j = kstep / g.src_width;
        const S* src = reinterpret_cast<const S*>(g.src[j]);
        const int off = k - j * g.src_width;
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) load_raw8<S>(st.a[u][mi], src + (size_t)arow[mi] * g.src_width + off);
      }
    }
  };

  f32x4 acc[MR];
#pragma unroll
  for (int mi = 0; mi < MR; ++mi) acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Stage<S, MR, PRO>& st) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bf16x8 wv = raw_to_bf16x8<S>(st.w[u]);
#pragma unroll
      for (int mi = 0; mi < MR; ++mi) {
        if constexpr (PRO == PRO_SPLIT) {
          acc[mi] = mfma16x16x32(wv, __builtin_bit_cast(bf16x8, st.a[u][mi].lo), acc[mi]);
          acc[mi] = mfma16x16x32(wv, __builtin_bit_cast(bf16x8, st.a[u][mi].hi), acc[mi]);
        } else if constexpr (sizeof(S) == 2) {
          acc[mi] = mfma16x16x32(wv, raw_to_bf16x8<S>(st.a[u][mi]), acc[mi]);
        } else {  // fp32 sources: split on the fly
          float f[8];
          raw_to_f32x8<S>(st.a[u][mi], f);
          bf16x8 hv;
          f32x4 l0, l1;
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[e] = (__bf16)f[e];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            l0[e] = f[e] - (float)hv[e];
            l1[e] = f[4 + e] - (float)hv[4 + e];
          }
          acc[mi] = mfma16x16x32(wv, hv, acc[mi]);
          acc[mi] = mfma16x16x32(wv, f32x8_to_bf16x8(l0, l1), acc[mi]);
        }
      }
    }
  };

  const int niter = g.kw / (32 * U);
  Stage<S, MR, PRO> s0, s1;
  if (niter > 0) fetch(s0, 0);

  // Row scale 1/rms from the producer's partial sums of squares (16 lanes per
  // row), computed while the first weight loads are in flight; it is applied
  // after the reduction below.
  if (row_scale) {
    for (int base = 0; base < MT * 16; base += nthr) {
      const int t = base + tid;
      const int m = t >> 4, part = t & 15;
      const int mm = min(m0 + m, g.M - 1);
      float ss = 0.f;
      if (m < MT)
        for (int p = part; p < g.ssq_nparts; p += 16) ss += g.ssq_in[p * g.ld_ssq + mm];
      ss += __shfl_xor(ss, 8);
      ss += __shfl_xor(ss, 4);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 1);
      if (part == 0 && m < MT) rinv_s[m] = 1.0f / sqrtf(ss / (float)g.K + g.eps);
    }
  }
  for (int it = 0; it < niter; it += 2) {
    if (it + 1 < niter) fetch(s1, it + 1);
    compute(s0);
    if (it + 1 < niter) {
      if (it + 2 < niter) fetch(s0, it + 2);
      compute(s1);
    }
  }

  // ---- partial tiles -> LDS, fixed-order reduction over WK, row scale
#pragma unroll
  for (int mi = 0; mi < MR; ++mi) {
    float* dst = red + ((wk * MT + 16 * mi + (lane & 15)) * NT + 16 * wn + 4 * (lane >> 4));
    *reinterpret_cast<f32x4*>(dst) = acc[mi];
  }
  __syncthreads();
  const int tsz = MT * NT;
  if (WK > 1 || row_scale) {
    for (int e = tid; e < tsz; e += nthr) {
      float v = red[e];
      for (int w = 1; w < WK; ++w) v += red[w * tsz + e];
      if (row_scale) v *= rinv_s[e / NT];
      red[e] = v;
    }
    __syncthreads();
  }

  // ---- epilogues: tile value of (row m0 + m, column tile_row(j)) is red[m * NT + j]
  if constexpr (EPI == EPI_F32_SSQ || EPI == EPI_RESID) {
    const float* src = red;
    const S* gn = reinterpret_cast<const S*>(g.gnext);
    bf16_t* oh = reinterpret_cast<bf16_t*>(g.out_hi);
    bf16_t* ol = reinterpret_cast<bf16_t*>(g.out_lo);
    if constexpr (EPI == EPI_RESID) {
      for (int e = tid; e < tsz; e += nthr) {
        const int m = e / NT, j = e - m * NT;
        if (m0 + m < g.M) red[e] += g.x[(size_t)(m0 + m) * g.N + tile_row(tile, j, NT, g.P)];
      }
      __syncthreads();
      if (g.conv != nullptr) {
        const S* cw = reinterpret_cast<const S*>(g.conv);
        for (int e = tid; e < tsz; e += nthr) {
          const int m = e / NT, j = e - m * NT;
          const int gm = m0 + m;
          if (gm >= g.M) continue;
          const int n = tile_row(tile, j, NT, g.P);
          const int i = gm % g.block;
          const float v = red[e];
          float y = load_f32<S>(cw + 3 * n + 1) * v;
          if (i > 0) y += load_f32<S>(cw + 3 * n) * red[e - NT];
          if (i < g.block - 1 && gm + 1 < g.M) y += load_f32<S>(cw + 3 * n + 2) * red[e + NT];
          aux[e] = v + y;
        }
        __syncthreads();
        src = aux;
      }
    }
    for (int e = tid; e < tsz; e += nthr) {
      const int m = e / NT, j = e - m * NT;
      if (m0 + m >= g.M) continue;
      const int n = tile_row(tile, j, NT, g.P);
      const size_t idx = (size_t)(m0 + m) * g.N + n;
      const float v = src[e];
      if constexpr (EPI == EPI_RESID) g.x[idx] = v;
      else g.out_f32[idx] = v;
      split_store(oh, ol, idx, v * load_f32<S>(gn + n));
    }
    // row sums of squares: 16 lanes per row
    for (int base = 0; base < MT * 16; base += nthr) {
      const int t = base + tid;
      const int m = t >> 4, part = t & 15;
      float s = 0.f;
      if (m < MT)
        for (int j = part; j < NT; j += 16) {
          const float v = src[m * NT + j];
          s += v * v;
        }
      s += __shfl_xor(s, 8);
      s += __shfl_xor(s, 4);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 1);
      if (part == 0 && m < MT && m0 + m < g.M) g.ssq_out[(size_t)tile * g.ld_ssq + m0 + m] = s;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int half = NT >> 1;
    const int F = g.N >> 1;
    bf16_t* oh = reinterpret_cast<bf16_t*>(g.out_hi);
    bf16_t* ol = reinterpret_cast<bf16_t*>(g.out_lo);
    for (int e = tid; e < MT * half; e += nthr) {
      const int m = e / half, jj = e - m * half;
      if (m0 + m >= g.M) continue;
      const int f = tile_row(tile, jj, NT, g.P);
      const float gv = red[m * NT + jj], uv = red[m * NT + jj + half];
      split_store(oh, ol, (size_t)(m0 + m) * F + f, silu_f32(gv) * uv);
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int half = NT >> 1;
    const int D = g.head_dim;
    const int Nq = g.n_q_heads * D, Nk = g.n_kv_heads * D;
    bf16_t* qh = reinterpret_cast<bf16_t*>(g.out_hi);
    bf16_t* ql = reinterpret_cast<bf16_t*>(g.out_lo);
    S* ko = reinterpret_cast<S*>(g.kb_out);
    S* vo = reinterpret_cast<S*>(g.vb_out);
    for (int e = tid; e < MT * half; e += nthr) {
      const int m = e / half, jj = e - m * half;
      const int gm = m0 + m;
      if (gm >= g.M) continue;
      const int n = tile_row(tile, jj, NT, g.P);  // d < D/2 of its head
      float lo = red[m * NT + jj], hi = red[m * NT + jj + half];
      const int pos = g.ctx_len[gm / g.block] + gm % g.block;
      if (n < Nq) {
        rope_pair(lo, hi, pos, n % D, D, g.rope_theta);
        split_store(qh, ql, (size_t)gm * Nq + n, lo * g.q_scale);
        split_store(qh, ql, (size_t)gm * Nq + n + D / 2, hi * g.q_scale);
      } else if (n < Nq + Nk) {
        const int nn = n - Nq;
        rope_pair(lo, hi, pos, nn % D, D, g.rope_theta);
        store_from_f32<S>(ko + (size_t)gm * Nk + nn, lo);
        store_from_f32<S>(ko + (size_t)gm * Nk + nn + D / 2, hi);
      } else {
        const int nn = n - Nq - Nk;
        store_from_f32<S>(vo + (size_t)gm * Nk + nn, lo);
        store_from_f32<S>(vo + (size_t)gm * Nk + nn + D / 2, hi);
      }
    }
  } else if constexpr (EPI == EPI_KV) {
    const int half = NT >> 1;
    const int D = g.head_dim, Hkv = g.n_kv_heads;
    const int seg_rows = Hkv * D;
    for (int e = tid; e < MT * half; e += nthr) {
      const int m = e / half, jj = e - m * half;
      const int gm = m0 + m;
      if (gm >= g.M) continue;
      const int b = gm / g.block, i = gm % g.block;
      const int t0 = g.ctx_len[b];
      if (t0 < 0 || t0 + g.block > g.max_ctx) {
        atomicOr(g.err, 1u);
        continue;
      }
      const int pos = t0 + i;
      const int n = tile_row(tile, jj, NT, g.P);
      const int seg = n / seg_rows, r = n - seg * seg_rows;
      const int head = r / D, d = r - head * D;
      float lo = red[m * NT + jj], hi = red[m * NT + jj + half];
      if ((seg & 1) == 0) rope_pair(lo, hi, pos, d, D, g.rope_theta);
      S* dst = reinterpret_cast<S*>(g.kv_cache[seg]) + (((size_t)b * g.max_ctx + pos) * Hkv + head) * D + d;
      store_from_f32<S>(dst, lo);
      store_from_f32<S>(dst + D / 2, hi);
    }
  } else if constexpr (EPI == EPI_ARGMAX) {
    if (g.logits_dbg != nullptr) {
      for (int e = tid; e < tsz; e += nthr) {
        const int m = e / NT, j = e - m * NT;
        if (m0 + m < g.M) g.logits_dbg[(size_t)(m0 + m) * g.N + tile_row(tile, j, NT, g.P)] = red[e];
      }
    }
    for (int base = 0; base < MT * 16; base += nthr) {
      const int t = base + tid;
      const int m = t >> 4, part = t & 15;
      uint64_t best = 0;
      if (m < MT)
        for (int j = part; j < NT; j += 16) {
          const uint64_t k = argmax_key(red[m * NT + j], (uint32_t)tile_row(tile, j, NT, g.P));
          best = k > best ? k : best;
        }
#pragma unroll
      for (int s = 8; s >= 1; s >>= 1) {
        const uint64_t o = shfl_xor_u64(best, s);
        best = o > best ? o : best;
      }
      if (part == 0 && m < MT && m0 + m < g.M) g.best_part[(size_t)tile * g.ld_best + m0 + m] = best;
    }
  }
}

// draft id of each row = index of the largest packed key over the LM-head tiles.
__global__ void __launch_bounds__(256) argmax_reduce_kernel(const uint64_t* part, int ntiles, int ld, int32_t* ids) {
  __shared__ uint64_t s_best[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  uint64_t best = 0;
  for (int t = tid; t < ntiles; t += 256) {
    const uint64_t k = part[(size_t)t * ld + m];
    best = k > best ? k : best;
  }
  best = wave_max_u64(best);
  if ((tid & 63) == 0) s_best[tid >> 6] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t b = s_best[0];
    for (int w = 1; w < 4; ++w) b = s_best[w] > b ? s_best[w] : b;
    ids[m] = argmax_key_index(b);
  }
}

hipError_t launch_argmax_reduce(const uint64_t* part, int ntiles, int ld, int M, int32_t* ids, hipStream_t stream) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(M), dim3(256), 0, stream, part, ntiles, ld, ids);
  return hipGetLastError();
}

int gemm_max_threads(int storage, ProKind pro, int MR) {
  return gemm_max_threads_for(pro == PRO_SPLIT || storage == ST_F32, MR);
}

size_t gemm_lds_bytes(EpiKind epi, int MR, int WN, int WK) {
  const size_t MT = 16 * MR, NT = 16 * WN;
  size_t b = (WK * MT * NT + MT) * sizeof(float);
  if (epi == EPI_RESID) b += MT * NT * sizeof(float);
  return b;
}

template <typename S, int MR, int PRO, int EPI>
static hipError_t launch_one(const GemmArgs& a, const GemmLaunch& l, hipStream_t stream) {
  dim3 grid(l.ntiles, l.mtiles), block(l.threads);
  hipLaunchKernelGGL((gemm_ws_kernel<S, MR, PRO, EPI>), grid, block, l.lds, stream, a);
  return hipGetLastError();
}

template <typename S, int PRO, int EPI>
static hipError_t launch_mr(const GemmArgs& a, const GemmLaunch& l, hipStream_t stream) {
  switch (l.MR) {
    case 1: return launch_one<S, 1, PRO, EPI>(a, l, stream);
    case 2: return launch_one<S, 2, PRO, EPI>(a, l, stream);
    case 4: return launch_one<S, 4, PRO, EPI>(a, l, stream);
    case 8: return launch_one<S, 8, PRO, EPI>(a, l, stream);
  }
  return hipErrorInvalidValue;
}

template <typename S>
static hipError_t launch_s(ProKind pro, EpiKind epi, const GemmArgs& a, const GemmLaunch& l, hipStream_t stream) {
  if (pro == PRO_CONCAT && epi == EPI_F32_SSQ) return launch_mr<S, PRO_CONCAT, EPI_F32_SSQ>(a, l, stream);
  if (pro == PRO_SPLIT && epi == EPI_KV) return launch_mr<S, PRO_SPLIT, EPI_KV>(a, l, stream);
  if (pro == PRO_SPLIT && epi == EPI_QKV) return launch_mr<S, PRO_SPLIT, EPI_QKV>(a, l, stream);
  if (pro == PRO_SPLIT && epi == EPI_RESID) return launch_mr<S, PRO_SPLIT, EPI_RESID>(a, l, stream);
  if (pro == PRO_SPLIT && epi == EPI_SWIGLU) return launch_mr<S, PRO_SPLIT, EPI_SWIGLU>(a, l, stream);
  if (pro == PRO_SPLIT && epi == EPI_ARGMAX) return launch_mr<S, PRO_SPLIT, EPI_ARGMAX>(a, l, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int storage, ProKind pro, EpiKind epi, const GemmArgs& a, const GemmLaunch& l,
                       hipStream_t stream) {
  if (storage == ST_BF16) return launch_s<bf16_t>(pro, epi, a, l, stream);
  return launch_s<float>(pro, epi, a, l, stream);
}

}  // namespace dfl
