// Non-causal grouped-query attention of a drafted block over
// [cached context ; the block itself], split over the key axis.
//
// One workgroup = (sequence b, KV head, key split) with 8 waves.  Its query
// rows are the G query heads of that KV head times the Bs block rows
// (QR = G*Bs rows, 16-row tiles); the waves are (query tile, key group)
// pairs, so with four query tiles two groups of four waves each take half of
// every 128-key stage and are merged through LDS at the end.  Every context
// K/V byte is read from HBM once per step, and all of a stage's K/V loads are
// issued together (one round of memory latency per stage).
//
// Scores are formed transposed (S^T = K Q^T, 16x16x32 MFMA) so that each lane
// owns one query row: the online-softmax max and scale are per lane, and the
// probabilities stay in registers and feed O^T = V^T P^T directly as the B
// operand.  V is stored transposed in LDS as key pairs (one dword = two keys
// of one dimension) with an XOR swizzle of the key-pair column by the
// dimension, which keeps the transposing stores at two-way bank conflicts and
// the operand reads conflict-free.  Queries and probabilities enter the bf16
// products as hi/lo pairs (two MFMAs each), keys and values as stored.
// Splits write unnormalised partials (O, running max, running sum) that a
// second kernel merges in a fixed order (deterministic; no cross-workgroup
// atomics, which cost tens of nanoseconds each on this chip).
#include "common.h"
#include "kernels.h"

namespace dfl {

constexpr int kStage = 128;   // keys per LDS stage
constexpr int kUnit = 32;     // keys per softmax update / PV product
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

template <int D>
struct AttnLds {
  static constexpr int KS = D + 8;        // K row stride (elements)
  static constexpr int VW = kStage / 2;   // V^T row length in dwords (key pairs)
  bf16_t k[kStage * KS];
  uint32_t vt[D * VW];
};

// Column of key pair kp in V^T row d.  Even, so a pair of key pairs stays
// adjacent and in order.
__device__ __forceinline__ int vt_col(int d, int kp) { return kp ^ (((d >> 3) ^ (d & 15)) << 1 & 30); }

__device__ __forceinline__ void split_out(bf16_t* hi, bf16_t* lo, size_t idx, float v) {
  const bf16_t h = f32_to_bf16_bits(v);
  hi[idx] = h;
  lo[idx] = f32_to_bf16_bits(v - bf16_bits_to_f32(h));
}

// Waves per key group (a power of two covering QT query tiles).
__host__ __device__ inline int attn_qtp(int QT) { return QT <= 1 ? 1 : QT <= 2 ? 2 : QT <= 4 ? 4 : 8; }

// QTP (waves per key group, >= the query tiles) is a template parameter so
// that a wave's key units unroll completely.
template <typename S, int D, int QTP>
__global__ void __launch_bounds__(kThreads) attention_kernel(const AttnArgs a) {
  constexpr int KG = kWaves / QTP < kStage / kUnit ? kWaves / QTP : kStage / kUnit;  // key groups
  constexpr int UPG = (kStage / kUnit) / KG;  // 32-key units per key group and stage
  extern __shared__ __align__(16) unsigned char lds_raw[];
  AttnLds<D>& L = *reinterpret_cast<AttnLds<D>*>(lds_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.z, kvh = blockIdx.y, sp = blockIdx.x;
  const int G = a.Hq / a.Hkv;
  const int QR = G * a.Bs;
  const int QT = (QR + 15) / 16;
  const int qt = wave % QTP, kg = wave / QTP;
  const bool computes = qt < QT && kg < KG;

  // ---- this lane's query row (loads issued before the context length arrives)
  const int r = 16 * qt + (lane & 15);
  const bool qvalid = computes && r < QR;
  const int rr = qvalid ? r : 0;
  const int gq = rr / a.Bs, iq = rr - gq * a.Bs;
  const int HqD = a.Hq * D;
  const size_t qoff = (size_t)(b * a.Bs + iq) * HqD + (kvh * G + gq) * D;
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

  // a caller-set length outside [0, max_ctx] is clamped so no access leaves the cache
  const int T = min(max(a.ctx_len[b], 0), a.max_ctx);
  const int total = T + a.Bs;
  const int ns = (total + a.CW - 1) / a.CW;
  if (sp >= ns) return;
  const int j0 = sp * a.CW;
  const int j1 = min(total, j0 + a.CW);
  const int nstages = (j1 - j0 + kStage - 1) / kStage;

  const S* kc = reinterpret_cast<const S*>(a.kc);
  const S* vc = reinterpret_cast<const S*>(a.vc);
  const S* kb = reinterpret_cast<const S*>(a.kb);
  const S* vb = reinterpret_cast<const S*>(a.vb);
  const size_t row = (size_t)a.Hkv * D;  // elements between consecutive keys
  auto key_ptr = [&](const S* cache, const S* blk, int j) {
    return j < T ? cache + ((size_t)b * a.max_ctx + j) * row + kvh * D
                 : blk + (size_t)(b * a.Bs + (j - T)) * row + kvh * D;
  };

  // ---- staging through registers.  K: (key, 8-dim piece) items, 16 lanes per
  // key row.  V: (key pair, piece) items; the two half-waves of 16 lanes take
  // key pairs 16 apart (the bank pattern the V^T swizzle is built for).
  constexpr int PIECES = D / 8;
  constexpr int KITEMS = kStage * PIECES;
  constexpr int VITEMS = (kStage / 2) * PIECES;
  constexpr int KPT = KITEMS / kThreads;
  constexpr int VPT = VITEMS / kThreads;
  static_assert(KITEMS % kThreads == 0 && VITEMS % kThreads == 0, "stage items must fill the workgroup");
  struct StageRegs {
    Raw8 k[KPT], v[VPT][2];
  };
  auto v_item = [&](int idx, int& kp, int& p) {
    p = idx % PIECES;
    const int h = (idx / PIECES) & 1, rest = idx / (2 * PIECES);
    kp = (rest & 15) + 16 * h + 32 * (rest >> 4);
  };
  // Loads are unconditional (keys past the split re-read its last key and are
  // zeroed at the store): branch-free address selects keep the loads of a
  // stage in flight together.
  auto stage_load = [&](StageRegs& R, int c0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * kThreads;
      const int key = idx / PIECES, p8 = (idx % PIECES) * 8;
      load_raw8<S>(R.k[i], key_ptr(kc, kb, min(c0 + key, j1 - 1)) + p8);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      int kp, p;
      v_item(tid + i * kThreads, kp, p);
#pragma unroll
      for (int t = 0; t < 2; ++t) load_raw8<S>(R.v[i][t], key_ptr(vc, vb, min(c0 + 2 * kp + t, j1 - 1)) + 8 * p);
    }
  };
  auto stage_store = [&](const StageRegs& R, int c0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * kThreads;
      const int key = idx / PIECES, p8 = (idx % PIECES) * 8;
      const bf16x8 v = c0 + key < j1 ? raw_to_bf16x8<S>(R.k[i]) : bf16x8{};
      *reinterpret_cast<bf16x8*>(&L.k[key * AttnLds<D>::KS + p8]) = v;
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      int kp, p;
      v_item(tid + i * kThreads, kp, p);
      float v0[8], v1[8];
      raw_to_f32x8<S>(R.v[i][0], v0);
      raw_to_f32x8<S>(R.v[i][1], v1);
      const bool ok0 = c0 + 2 * kp < j1, ok1 = c0 + 2 * kp + 1 < j1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * p + e;
        const uint32_t lo = ok0 ? (uint32_t)f32_to_bf16_bits(v0[e]) : 0u;
        const uint32_t hi = ok1 ? (uint32_t)f32_to_bf16_bits(v1[e]) : 0u;
        L.vt[d * AttnLds<D>::VW + vt_col(d, kp)] = lo | (hi << 16);
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) o[ds] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stages are fetched PF ahead through a pair of register sets: with PF = 2
  // the loads of stage st+2 are issued before the matrix work of stage st and
  // stage st+1 (fetched a stage earlier) is stored to LDS after it; the widest
  // wave layout (eight query tiles) and fp32 storage need the registers and
  // fetch one ahead.
  constexpr int PF = (QTP >= 8 || sizeof(S) == 4) ? 1 : 2;
  StageRegs ra, rb;
  stage_load(ra, j0);
  if (PF == 2 && nstages > 1) stage_load(rb, j0 + kStage);
  stage_store(ra, j0);
  __syncthreads();
  auto step = [&](StageRegs& fr, StageRegs& nx, int st) {
    const int c0 = j0 + st * kStage;
    if (PF == 2 && st + 2 < nstages) stage_load(fr, c0 + 2 * kStage);  // fr's stage st is already in LDS
    if (PF == 1 && st + 1 < nstages) stage_load(nx, c0 + kStage);
    if (computes) {
      // ---- scores S^T[key][q] of all the wave's units (independent MFMA
      // chains), then one softmax update and one rescale for the stage
      f32x4 sc[UPG][2];
#pragma unroll
      for (int uu = 0; uu < UPG; ++uu) {
        const int u = kg * UPG + uu;
#pragma unroll
        for (int h = 0; h < 2; ++h) sc[uu][h] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c0 + kUnit * u >= j1) continue;
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
                &L.k[(kUnit * u + 16 * h + (lane & 15)) * AttnLds<D>::KS + 32 * s + 8 * (lane >> 4)]);
            sc[uu][h] = mfma16x16x32(kf, qf[s], sc[uu][h]);
            sc[uu][h] = mfma16x16x32(kf, qr[s], sc[uu][h]);
          }
      }
      // lane holds keys c0 + 32*u + 16*h + 4*(lane>>4) + e for query row (lane & 15)
      float cmax = -INFINITY;
#pragma unroll
      for (int uu = 0; uu < UPG; ++uu)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (c0 + kUnit * (kg * UPG + uu) + 16 * h + 4 * (lane >> 4) + e >= j1) sc[uu][h][e] = -INFINITY;
            cmax = fmaxf(cmax, sc[uu][h][e]);
          }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      const float m_new = fmaxf(m_run, cmax);
      if (m_new != -INFINITY) {  // some key of this wave's share of the stage is valid
        const float alpha = fast_exp2(m_run - m_new);
        float psum = 0.f;
#pragma unroll
        for (int uu = 0; uu < UPG; ++uu)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sc[uu][h][e] = fast_exp2(sc[uu][h][e] - m_new);
              psum += sc[uu][h][e];
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) o[ds] *= alpha;
        // ---- O^T[d][q] += V^T[d][keys] P^T[keys][q]; P as a hi/lo pair
#pragma unroll
        for (int uu = 0; uu < UPG; ++uu) {
          const int u = kg * UPG + uu;
          if (c0 + kUnit * u >= j1) continue;
          bf16x8 ph, pl;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ph[e] = (__bf16)sc[uu][0][e];
            ph[4 + e] = (__bf16)sc[uu][1][e];
            pl[e] = (__bf16)(sc[uu][0][e] - (float)ph[e]);
            pl[4 + e] = (__bf16)(sc[uu][1][e] - (float)ph[4 + e]);
          }
          const int kp0 = (kUnit / 2) * u + 2 * (lane >> 4);  // keys 32*u + 4*(lane>>4) + [0, 4)
#pragma unroll
          for (int ds = 0; ds < D / 16; ++ds) {
            const int d = 16 * ds + (lane & 15);
            const uint32_t* vrow = &L.vt[d * AttnLds<D>::VW];
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + vt_col(d, kp0));
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + vt_col(d, kp0 + 8));
            const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
            o[ds] = mfma16x16x32(vf, ph, o[ds]);
            o[ds] = mfma16x16x32(vf, pl, o[ds]);
          }
        }
      }
    }
    if (st + 1 < nstages) {
      __syncthreads();
      stage_store(nx, c0 + kStage);
      __syncthreads();
    }
  };
  if constexpr (PF == 1) {
    for (int st = 0; st < nstages; ++st) step(ra, ra, st);
  } else {
    for (int st = 0; st < nstages; st += 2) {
      step(ra, rb, st);
      if (st + 1 < nstages) step(rb, ra, st + 1);
    }
  }

  // ---- merge the key groups of each query tile through LDS (group 0 keeps the
  // result).  Records are [group-1][tile][d-slice][lane] 16-byte slots, so a
  // wave's LDS traffic is conflict-free 16-byte accesses.
  if constexpr (KG > 1) {
    __syncthreads();  // every wave is done reading K / V^T
    f32x4* mo = reinterpret_cast<f32x4*>(lds_raw);                       // [KG-1][QTP][D/16][64]
    float* mml = reinterpret_cast<float*>(mo + (KG - 1) * QTP * (D / 16) * 64);  // [KG-1][QTP][64][2]
    if (computes && kg > 0) {
      const int g = (kg - 1) * QTP + qt;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) mo[(g * (D / 16) + ds) * 64 + lane] = o[ds];
      mml[(g * 64 + lane) * 2] = m_run;
      mml[(g * 64 + lane) * 2 + 1] = l_run;
    }
    __syncthreads();
    if (computes && kg == 0) {
#pragma unroll
      for (int g2 = 1; g2 < KG; ++g2) {
        const int g = (g2 - 1) * QTP + qt;
        const float m2 = mml[(g * 64 + lane) * 2], l2 = mml[(g * 64 + lane) * 2 + 1];
        const float mn = fmaxf(m_run, m2);  // finite: group 0 always has a valid key
        const float w1 = fast_exp2(m_run - mn);
        const float w2 = m2 == -INFINITY ? 0.f : fast_exp2(m2 - mn);
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) o[ds] = o[ds] * w1 + mo[(g * (D / 16) + ds) * 64 + lane] * w2;
        l_run = l_run * w1 + l2 * w2;
        m_run = mn;
      }
    }
  }
  if (!computes || kg != 0) return;

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

// Merge of the split partials of one (sequence, KV head).  A wave covers four
// (query row, 4 dims) items; its 16 lane groups take splits g, g+16, ... so all
// partial loads are issued together, and the groups are folded by a fixed
// butterfly (deterministic).  grid: (item groups of 16, Hkv, B), 256 threads.
template <int D>
__global__ void __launch_bounds__(256) attention_combine_kernel(const AttnArgs a) {
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int T = min(max(a.ctx_len[b], 0), a.max_ctx);
  const int ns = (T + a.Bs + a.CW - 1) / a.CW;
  if (ns <= 1) return;  // written directly by the split kernel
  const int G = a.Hq / a.Hkv;
  const int QR = G * a.Bs;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sg = lane >> 2;
  const int item = blockIdx.x * 16 + wave * 4 + (lane & 3);
  const bool valid = item < QR * (D / 4);
  const int it = valid ? item : 0;
  const int r = it / (D / 4), d4 = (it - r * (D / 4)) * 4;
  const size_t pbase = ((size_t)(b * a.Hkv + kvh) * a.max_splits);
  const float* ml = a.part_ml + (pbase * QR + r) * 2;
  const float* po = a.part_o + (pbase * QR + r) * D + d4;
  const size_t sstride_ml = (size_t)QR * 2, sstride_o = (size_t)QR * D;

  float m = -INFINITY, l = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += 64) {
    float mv[4], lv[4];
    f32x4 ov[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = s0 + sg + 16 * k;
      mv[k] = -INFINITY;
      lv[k] = 0.f;
      ov[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s < ns) {
        mv[k] = ml[s * sstride_ml];
        lv[k] = ml[s * sstride_ml + 1];
        ov[k] = *reinterpret_cast<const f32x4*>(po + s * sstride_o);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float mn = fmaxf(m, mv[k]);
      if (mn == -INFINITY) continue;
      const float w1 = m == -INFINITY ? 0.f : fast_exp2(m - mn);
      const float w2 = mv[k] == -INFINITY ? 0.f : fast_exp2(mv[k] - mn);
      acc = acc * w1 + ov[k] * w2;
      l = l * w1 + lv[k] * w2;
      m = mn;
    }
  }
#pragma unroll
  for (int x = 4; x <= 32; x <<= 1) {
    const float mo = __shfl_xor(m, x), lo = __shfl_xor(l, x);
    f32x4 ao;
#pragma unroll
    for (int e = 0; e < 4; ++e) ao[e] = __shfl_xor(acc[e], x);
    const float mn = fmaxf(m, mo);
    const float w1 = m == -INFINITY ? 0.f : fast_exp2(m - mn);
    const float w2 = mo == -INFINITY ? 0.f : fast_exp2(mo - mn);
    acc = acc * w1 + ao * w2;
    l = l * w1 + lo * w2;
    m = mn;
  }
  if (sg != 0 || !valid) return;
  const float inv = 1.0f / l;
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
  if (QR > 16 * kWaves || a.CW <= 0 || a.CW % 16) return hipErrorInvalidValue;
  const size_t lds = sizeof(AttnLds<D>);
  const int qtp = attn_qtp((QR + 15) / 16);
  auto k = qtp == 1 ? attention_kernel<S, D, 1>
                    : qtp == 2 ? attention_kernel<S, D, 2> : qtp == 4 ? attention_kernel<S, D, 4> : attention_kernel<S, D, 8>;
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
  hipLaunchKernelGGL(k, dim3(a.max_splits, a.Hkv, a.batch), dim3(kThreads), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits <= 1) return e;
  const int items = QR * (D / 4);
  hipLaunchKernelGGL(attention_combine_kernel<D>, dim3((items + 15) / 16, a.Hkv, a.batch), dim3(256), 0, stream, a);
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
