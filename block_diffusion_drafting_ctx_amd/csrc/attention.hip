// Non-causal grouped-query attention of a drafted block over
// [cached context ; the block itself], split over the key axis.
//
// One workgroup = (sequence b, KV head, key split).  Its query rows are the
// G query heads of that KV head times the Bs block rows (QR = G*Bs rows,
// one 16-row tile per compute wave), so every context K/V byte is read from
// HBM once per step.  Keys stream through LDS in chunks of 64, double
// buffered: the next chunk's K/V loads are in flight (in registers) while the
// current chunk is consumed, with one barrier per chunk.  Scores are formed
// transposed (S^T = K Q^T, 16x16x32 MFMA) so that each lane owns one query
// row: the online-softmax max and scale are per lane, and the probabilities
// stay in registers and feed O^T = V^T P^T directly as the B operand (V is
// stored transposed in LDS).  Queries and probabilities enter the bf16
// products as hi/lo pairs (two MFMAs each), keys and values as stored.
// Splits write unnormalised partials (O, running max, running sum) that a
// second kernel merges in split order (deterministic; no cross-workgroup
// atomics, which cost tens of nanoseconds each on this chip).
#include "common.h"
#include "kernels.h"

namespace dfl {

constexpr int kChunk = 64;  // keys per LDS stage

template <int D>
struct AttnLds {
  static constexpr int KS = D + 8;       // K row stride (elements)
  static constexpr int VS = kChunk + 8;  // V^T row stride (elements)
  bf16_t k[kChunk * KS];
  bf16_t vt[D * VS];
};

__device__ __forceinline__ void split_out(bf16_t* hi, bf16_t* lo, size_t idx, float v) {
  const bf16_t h = f32_to_bf16_bits(v);
  hi[idx] = h;
  lo[idx] = f32_to_bf16_bits(v - bf16_bits_to_f32(h));
}

// Threads of an attention workgroup: one wave per 16 query rows, at least four
// (the extra waves only help staging).
__host__ __device__ inline int attn_threads(int QR) {
  const int w = (QR + 15) / 16;
  return 64 * (w < 4 ? 4 : w);
}

template <typename S, int D>
__global__ void __launch_bounds__(512) attention_kernel(const AttnArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  AttnLds<D>* lds = reinterpret_cast<AttnLds<D>*>(lds_raw);  // [2]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x;
  const int b = blockIdx.z, kvh = blockIdx.y, sp = blockIdx.x;
  const int G = a.Hq / a.Hkv;
  const int QR = G * a.Bs;
  const int QT = (QR + 15) / 16;

  // a caller-set length outside [0, max_ctx] is clamped so no access leaves the cache
  const int T = min(max(a.ctx_len[b], 0), a.max_ctx);
  const int total = T + a.Bs;
  const int ns = (total + a.CW - 1) / a.CW;
  if (sp >= ns) return;
  const int j0 = sp * a.CW;
  const int j1 = min(total, j0 + a.CW);
  const int nchunks = (j1 - j0 + kChunk - 1) / kChunk;

  // ---- this lane's query row
  const int r = 16 * wave + (lane & 15);
  const bool computes = wave < QT;
  const bool qvalid = r < QR;
  const int rr = qvalid ? r : 0;
  const int gq = rr / a.Bs, iq = rr - gq * a.Bs;
  const int h = kvh * G + gq;
  const int HqD = a.Hq * D;
  const size_t qoff = (size_t)(b * a.Bs + iq) * HqD + h * D;
  bf16x8 qf[D / 32], qr[D / 32];  // query = qf + qr (hi/lo pair)
  {
    const bf16_t* qh = reinterpret_cast<const bf16_t*>(a.q_hi) + qoff;
    const bf16_t* ql = reinterpret_cast<const bf16_t*>(a.q_lo) + qoff;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      qf[s] = bf16x8{};
      qr[s] = bf16x8{};
      if (qvalid) {
        qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + 32 * s + 8 * (lane >> 4)));
        qr[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ql + 32 * s + 8 * (lane >> 4)));
      }
    }
  }

  const S* kc = reinterpret_cast<const S*>(a.kc);
  const S* vc = reinterpret_cast<const S*>(a.vc);
  const S* kb = reinterpret_cast<const S*>(a.kb);
  const S* vb = reinterpret_cast<const S*>(a.vb);
  const size_t row = (size_t)a.Hkv * D;  // elements between consecutive keys
  auto key_ptr = [&](const S* cache, const S* blk, int j) {
    return j < T ? cache + ((size_t)b * a.max_ctx + j) * row + kvh * D
                 : blk + (size_t)(b * a.Bs + (j - T)) * row + kvh * D;
  };

  // ---- staging through registers: K as 8-element pieces, V as key pairs
  constexpr int PIECES = D / 8;
  constexpr int KITEMS = kChunk * PIECES;        // K pieces per chunk
  constexpr int VITEMS = (kChunk / 2) * PIECES;  // V key-pair pieces per chunk
  constexpr int KPT = (KITEMS + 255) / 256;      // per thread (workgroups have >= 256 threads)
  constexpr int VPT = (VITEMS + 255) / 256;
  Raw8 kreg[KPT], vreg[VPT][2];
  auto stage_load = [&](int c0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * nthr;
      if (idx < KITEMS) {
        const int key = idx / PIECES, p8 = (idx - key * PIECES) * 8;
        const int j = c0 + key;
        if (j < j1) load_raw8<S>(kreg[i], key_ptr(kc, kb, j) + p8);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * nthr;
      if (idx < VITEMS) {
        const int kp = idx / PIECES, p8 = (idx - kp * PIECES) * 8;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int j = c0 + 2 * kp + t;
          if (j < j1) load_raw8<S>(vreg[i][t], key_ptr(vc, vb, j) + p8);
        }
      }
    }
  };
  auto stage_store = [&](AttnLds<D>& L, int c0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * nthr;
      if (idx < KITEMS) {
        const int key = idx / PIECES, p8 = (idx - key * PIECES) * 8;
        const bf16x8 v = c0 + key < j1 ? raw_to_bf16x8<S>(kreg[i]) : bf16x8{};
        *reinterpret_cast<bf16x8*>(&L.k[key * AttnLds<D>::KS + p8]) = v;
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * nthr;
      if (idx < VITEMS) {
        const int kp = idx / PIECES, p8 = (idx - kp * PIECES) * 8;
        float v0[8], v1[8];
        raw_to_f32x8<S>(vreg[i][0], v0);
        raw_to_f32x8<S>(vreg[i][1], v1);
        const bool ok0 = c0 + 2 * kp < j1, ok1 = c0 + 2 * kp + 1 < j1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t lo = ok0 ? (uint32_t)f32_to_bf16_bits(v0[e]) : 0u;
          const uint32_t hi = ok1 ? (uint32_t)f32_to_bf16_bits(v1[e]) : 0u;
          *reinterpret_cast<uint32_t*>(&L.vt[(p8 + e) * AttnLds<D>::VS + 2 * kp]) = lo | (hi << 16);
        }
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) o[ds] = f32x4{0.f, 0.f, 0.f, 0.f};

  stage_load(j0);
  stage_store(lds[0], j0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int c0 = j0 + c * kChunk;
    AttnLds<D>& L = lds[c & 1];
    if (c + 1 < nchunks) stage_load(c0 + kChunk);  // in flight during this chunk
    if (computes) {
      // ---- scores S^T[key][q] for 4 key subtiles of 16
      f32x4 sc[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        sc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
              &L.k[(16 * st + (lane & 15)) * AttnLds<D>::KS + 32 * s + 8 * (lane >> 4)]);
          sc[st] = mfma16x16x32(kf, qf[s], sc[st]);
          sc[st] = mfma16x16x32(kf, qr[s], sc[st]);
        }
      }
      // lane holds keys c0 + 16*st + 4*(lane>>4) + e for query row (lane & 15)
      float cmax = -INFINITY;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = c0 + 16 * st + 4 * (lane >> 4) + e;
          if (j >= j1) sc[st][e] = -INFINITY;
          cmax = fmaxf(cmax, sc[st][e]);
        }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = fast_exp2(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc[st][e] = fast_exp2(sc[st][e] - m_new);
          psum += sc[st][e];
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) o[ds] *= alpha;

      // ---- O^T[d][q] += V^T[d][keys] P^T[keys][q], 32 keys per product; P as a hi/lo pair
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 ph, pl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ph[e] = (__bf16)sc[2 * t][e];
          ph[4 + e] = (__bf16)sc[2 * t + 1][e];
          pl[e] = (__bf16)(sc[2 * t][e] - (float)ph[e]);
          pl[4 + e] = (__bf16)(sc[2 * t + 1][e] - (float)ph[4 + e]);
        }
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
          const bf16_t* vrow = &L.vt[(16 * ds + (lane & 15)) * AttnLds<D>::VS + 32 * t + 4 * (lane >> 4)];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          o[ds] = mfma16x16x32(vf, ph, o[ds]);
          o[ds] = mfma16x16x32(vf, pl, o[ds]);
        }
      }
    }
    if (c + 1 < nchunks) stage_store(lds[(c + 1) & 1], c0 + kChunk);
    __syncthreads();
  }
  if (!computes) return;

  // lane (q = lane & 15) holds O^T rows d = 16*ds + 4*(lane>>4) + e
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);

  if (ns == 1) {
    if (qvalid) {
      bf16_t* out_h = reinterpret_cast<bf16_t*>(a.out_hi);
      bf16_t* out_l = reinterpret_cast<bf16_t*>(a.out_lo);
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
        for (int e = 0; e < 4; ++e) split_out(out_h, out_l, qoff + 16 * ds + 4 * (lane >> 4) + e, o[ds][e] * inv);
    }
    return;
  }
  const size_t pbase = ((size_t)(b * a.Hkv + kvh) * a.max_splits);
  if (qvalid) {
    float* po = a.part_o + ((pbase + sp) * QR + r) * D;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) *reinterpret_cast<f32x4*>(po + 16 * ds + 4 * (lane >> 4)) = o[ds];
    if ((lane >> 4) == 0) {
      a.part_ml[((pbase + sp) * QR + r) * 2 + 0] = m_run;
      a.part_ml[((pbase + sp) * QR + r) * 2 + 1] = l_tot;
    }
  }
}

// Merge of the split partials of one (sequence, KV head): one thread per
// (query row, 4 dims), splits folded in split order.  grid: (row-chunks, Hkv, B).
template <int D>
__global__ void __launch_bounds__(256) attention_combine_kernel(const AttnArgs a) {
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int T = min(max(a.ctx_len[b], 0), a.max_ctx);
  const int ns = (T + a.Bs + a.CW - 1) / a.CW;
  if (ns <= 1) return;  // written directly by the split kernel
  const int G = a.Hq / a.Hkv;
  const int QR = G * a.Bs;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= QR * (D / 4)) return;
  const int r = idx / (D / 4), d4 = (idx - r * (D / 4)) * 4;
  const size_t pbase = ((size_t)(b * a.Hkv + kvh) * a.max_splits);
  const float* ml = a.part_ml + (pbase * QR + r) * 2;
  const float* po = a.part_o + (pbase * QR + r) * D + d4;
  const size_t sstride_ml = (size_t)QR * 2, sstride_o = (size_t)QR * D;
  float mx = -INFINITY;
#pragma unroll 4
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, ml[s * sstride_ml]);
  float lsum = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = 0; s < ns; ++s) {
    const float wgt = fast_exp2(ml[s * sstride_ml] - mx);
    lsum += ml[s * sstride_ml + 1] * wgt;
    acc += *reinterpret_cast<const f32x4*>(po + s * sstride_o) * wgt;
  }
  const float inv = 1.0f / lsum;
  const int gq = r / a.Bs, iq = r - gq * a.Bs;
  const size_t orow = (size_t)(b * a.Bs + iq) * (a.Hq * D) + (kvh * G + gq) * D + d4;
  bf16_t* out_h = reinterpret_cast<bf16_t*>(a.out_hi);
  bf16_t* out_l = reinterpret_cast<bf16_t*>(a.out_lo);
#pragma unroll
  for (int e = 0; e < 4; ++e) split_out(out_h, out_l, orow + e, acc[e] * inv);
}

template <typename S, int D>
static hipError_t launch_attention_d(const AttnArgs& a, hipStream_t stream) {
  const int QR = (a.Hq / a.Hkv) * a.Bs;
  const size_t lds = 2 * sizeof(AttnLds<D>);
  auto k = attention_kernel<S, D>;
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
  hipLaunchKernelGGL(k, dim3(a.max_splits, a.Hkv, a.batch), dim3(attn_threads(QR)), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits <= 1) return e;
  const int nthreads = QR * (D / 4);
  hipLaunchKernelGGL(attention_combine_kernel<D>, dim3((nthreads + 255) / 256, a.Hkv, a.batch), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

template <typename S>
static hipError_t launch_attention_s(const AttnArgs& a, hipStream_t stream) {
  if (a.D == 128) return launch_attention_d<S, 128>(a, stream);
  if (a.D == 64) return launch_attention_d<S, 64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attention(int storage, const AttnArgs& a, hipStream_t stream) {
  if (storage == ST_BF16) return launch_attention_s<bf16_t>(a, stream);
  return launch_attention_s<float>(a, stream);
}

}  // namespace dfl
