// Non-causal grouped-query attention of a drafted block over
// [cached context ; the block itself], split over the key axis.
//
// One workgroup = (sequence b, KV head, key split).  Its query rows are the
// G query heads of that KV head times the Bs block rows (QR = G*Bs rows,
// one 16-row tile per wave), so every context K/V byte is read from HBM once
// per step.  Per 64-key chunk the keys are staged to LDS (K as rows, V
// transposed), scores are formed transposed (S^T = K Q^T, 16x16x32 MFMA) so
// that each lane owns one query row: the online-softmax max and scale are
// per lane, the probabilities stay in registers and feed the second product
// O^T = V^T P^T directly as the B operand.  Queries and probabilities enter
// the bf16 products as hi/lo pairs (two MFMAs each), keys and values as
// stored; the output is written as a hi/lo pair for the output projection.  Splits write unnormalised
// partials (O, running max, running sum) that a second kernel merges in
// split order (deterministic; no cross-workgroup atomics, which cost tens of
// nanoseconds each on this chip).
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

template <typename S, int D>
__global__ void __launch_bounds__(512) attention_kernel(const AttnArgs a) {
  __shared__ AttnLds<D> lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x;
  const int b = blockIdx.z, kvh = blockIdx.y, sp = blockIdx.x;
  const int G = a.Hq / a.Hkv;
  const int QR = G * a.Bs;

  // a caller-set length outside [0, max_ctx] is clamped so no access leaves the cache
  const int T = min(max(a.ctx_len[b], 0), a.max_ctx);
  const int total = T + a.Bs;
  const int ns = (total + a.CW - 1) / a.CW;
  if (sp >= ns) return;
  const int j0 = sp * a.CW;
  const int j1 = min(total, j0 + a.CW);

  // ---- this lane's query row
  const int r = 16 * wave + (lane & 15);
  const bool qvalid = r < QR;
  const int rr = qvalid ? r : 0;
  const int gq = rr / a.Bs, iq = rr - gq * a.Bs;
  const int h = kvh * G + gq;
  const int HqD = a.Hq * D;
  const size_t qoff = (size_t)(b * a.Bs + iq) * HqD + h * D;
  const bf16_t* qh = reinterpret_cast<const bf16_t*>(a.q_hi) + qoff;
  const bf16_t* ql = reinterpret_cast<const bf16_t*>(a.q_lo) + qoff;
  bf16x8 qf[D / 32], qr[D / 32];  // query = qf + qr (hi/lo pair)
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + 32 * s + 8 * (lane >> 4)));
    qr[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ql + 32 * s + 8 * (lane >> 4)));
    if (!qvalid) {
      qf[s] = bf16x8{};
      qr[s] = bf16x8{};
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) o[ds] = f32x4{0.f, 0.f, 0.f, 0.f};

  const S* kc = reinterpret_cast<const S*>(a.kc);
  const S* vc = reinterpret_cast<const S*>(a.vc);
  const S* kb = reinterpret_cast<const S*>(a.kb);
  const S* vb = reinterpret_cast<const S*>(a.vb);
  const size_t ctx_row = (size_t)a.Hkv * D;  // elements between consecutive cached keys

  for (int c0 = j0; c0 < j1; c0 += kChunk) {
    // ---- stage K rows: one 8-element piece per item
    constexpr int PIECES = D / 8;
    for (int idx = tid; idx < kChunk * PIECES; idx += nthr) {
      const int key = idx / PIECES, p8 = (idx - key * PIECES) * 8;
      const int j = c0 + key;
      bf16x8 v = bf16x8{};
      if (j < j1) {
        const S* src = j < T ? kc + ((size_t)b * a.max_ctx + j) * ctx_row + kvh * D
                             : kb + ((size_t)(b * a.Bs + (j - T))) * ctx_row + kvh * D;
        Raw8 raw;
        load_raw8<S>(raw, src + p8);
        v = raw_to_bf16x8<S>(raw);
      }
      *reinterpret_cast<bf16x8*>(&lds.k[key * AttnLds<D>::KS + p8]) = v;
    }
    // ---- stage V transposed: key pairs, 8 dims per item, 4-byte LDS stores
    for (int idx = tid; idx < (kChunk / 2) * PIECES; idx += nthr) {
      const int kp = idx / PIECES, p8 = (idx - kp * PIECES) * 8;
      float v0[8], v1[8];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int j = c0 + 2 * kp + t;
        float* dstf = t ? v1 : v0;
        if (j < j1) {
          const S* src = j < T ? vc + ((size_t)b * a.max_ctx + j) * ctx_row + kvh * D
                               : vb + ((size_t)(b * a.Bs + (j - T))) * ctx_row + kvh * D;
          Raw8 raw;
          load_raw8<S>(raw, src + p8);
          raw_to_f32x8<S>(raw, dstf);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) dstf[e] = 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t pk = (uint32_t)f32_to_bf16_bits(v0[e]) | ((uint32_t)f32_to_bf16_bits(v1[e]) << 16);
        *reinterpret_cast<uint32_t*>(&lds.vt[(p8 + e) * AttnLds<D>::VS + 2 * kp]) = pk;
      }
    }
    __syncthreads();

    // ---- scores S^T[key][q] for 4 key subtiles of 16
    f32x4 sc[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      sc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            &lds.k[(16 * st + (lane & 15)) * AttnLds<D>::KS + 32 * s + 8 * (lane >> 4)]);
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
        const bf16_t* vrow = &lds.vt[(16 * ds + (lane & 15)) * AttnLds<D>::VS + 32 * t + 4 * (lane >> 4)];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        o[ds] = mfma16x16x32(vf, ph, o[ds]);
        o[ds] = mfma16x16x32(vf, pl, o[ds]);
      }
    }
    __syncthreads();
  }

  // lane (q = lane & 15) holds O^T rows d = 16*ds + 4*(lane>>4) + e
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  bf16_t* out_h = reinterpret_cast<bf16_t*>(a.out_hi);
  bf16_t* out_l = reinterpret_cast<bf16_t*>(a.out_lo);
  const size_t orow = qoff;

  if (ns == 1) {
    if (qvalid) {
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
        for (int e = 0; e < 4; ++e) split_out(out_h, out_l, orow + 16 * ds + 4 * (lane >> 4) + e, o[ds][e] * inv);
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

// Merge of the split partials of one (sequence, KV head): in split order, so
// the result does not depend on which split finished first.
template <int D>
__global__ void __launch_bounds__(256) attention_combine_kernel(const AttnArgs a) {
  const int b = blockIdx.y, kvh = blockIdx.x;
  const int T = min(max(a.ctx_len[b], 0), a.max_ctx);
  const int ns = (T + a.Bs + a.CW - 1) / a.CW;
  if (ns <= 1) return;  // written directly by the split kernel
  const int G = a.Hq / a.Hkv;
  const int QR = G * a.Bs;
  const int HqD = a.Hq * D;
  const size_t pbase = ((size_t)(b * a.Hkv + kvh) * a.max_splits);
  bf16_t* out_h = reinterpret_cast<bf16_t*>(a.out_hi);
  bf16_t* out_l = reinterpret_cast<bf16_t*>(a.out_lo);
  for (int idx = threadIdx.x; idx < QR * (D / 4); idx += blockDim.x) {
    const int r = idx / (D / 4), d4 = (idx - r * (D / 4)) * 4;
    float mx = -INFINITY;
    for (int s = 0; s < ns; ++s) mx = fmaxf(mx, a.part_ml[((pbase + s) * QR + r) * 2]);
    float lsum = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ns; ++s) {
      const float* ml = a.part_ml + ((pbase + s) * QR + r) * 2;
      const float wgt = fast_exp2(ml[0] - mx);
      lsum += ml[1] * wgt;
      acc += *reinterpret_cast<const f32x4*>(a.part_o + ((pbase + s) * QR + r) * D + d4) * wgt;
    }
    const float inv = 1.0f / lsum;
    const int gq = r / a.Bs, iq = r - gq * a.Bs;
    const size_t orow = (size_t)(b * a.Bs + iq) * HqD + (kvh * G + gq) * D + d4;
#pragma unroll
    for (int e = 0; e < 4; ++e) split_out(out_h, out_l, orow + e, acc[e] * inv);
  }
}

template <typename S>
static hipError_t launch_attention_s(const AttnArgs& a, hipStream_t stream) {
  const int QR = (a.Hq / a.Hkv) * a.Bs;
  const int waves = (QR + 15) / 16;
  dim3 grid(a.max_splits, a.Hkv, a.batch), block(64 * waves);
  if (a.D == 128)
    hipLaunchKernelGGL((attention_kernel<S, 128>), grid, block, 0, stream, a);
  else if (a.D == 64)
    hipLaunchKernelGGL((attention_kernel<S, 64>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits <= 1) return e;
  if (a.D == 128)
    hipLaunchKernelGGL((attention_combine_kernel<128>), dim3(a.Hkv, a.batch), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((attention_combine_kernel<64>), dim3(a.Hkv, a.batch), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attention(int storage, const AttnArgs& a, hipStream_t stream) {
  if (storage == ST_BF16) return launch_attention_s<bf16_t>(a, stream);
  return launch_attention_s<float>(a, stream);
}

}  // namespace dfl
