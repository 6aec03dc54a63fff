// Non-causal grouped-query attention of a drafted block over
// [cached context ; the block itself], with the key axis of the whole batch
// cut evenly over the compute units.
//
// Every key is read from this layer's cache: the block's own K/V rows sit at
// cache rows T_b + i (staged there by the Q/K/V finish kernel), so key j of
// (sequence b, KV head h) is cache row j for j < L_b = T_b + Bs, and a key's
// address never depends on T_b -- only whether it counts does.
//
// Work decomposition.  Every (b, h) pair is a segment of L_b keys; the parts
// of segments the workgroups own are pieces.
//  * Fixed chunks (small batches; chosen by the host): every segment is cut
//    at multiples of a chunk size C fixed from the cache capacity, so
//    workgroup (segment, chunk) knows its keys and queries from its index and
//    issues its query, K/V and context-length loads together; chunks past L_b
//    are dropped once the length arrives.
//  * Planned (large batches): from the context lengths each workgroup builds
//    the plan in LDS.  Either every segment is cut into a number of balanced
//    pieces in proportion to its length (one workgroup each), or the segments
//    are laid end to end (b major, h minor) and the resulting key axis is cut
//    into gridDim.x equal ranges, where a workgroup closes its piece at a
//    segment end and starts the next one with that segment's queries.
// A workgroup walks its range in stages of 192 keys.  A piece that is a whole
// segment writes the normalised output; any other piece writes an
// unnormalised partial (O, running max, running sum) into slot w + s
// (workgroup w, segment s: distinct for every piece, since a later piece of
// the same workgroup has a larger segment index and a later piece of the same
// segment a larger workgroup index), and a second kernel merges the pieces of
// each split segment in a fixed order (deterministic; no cross-workgroup
// atomics).  All of it runs in one dispatch round.
//
// Two forms compute a piece.  A bf16 cache streams through an LDS ring fed
// by LDS-DMA loads in MFMA fragment order, V read through the transposing
// LDS read (attention_ring_kernel, below).  An fp32 or 8-bit cache takes the
// register-staged form described next, which converts while it stores.
//
// Inside a piece: one workgroup of 8 waves; its query rows are the G query
// heads of the KV head times the Bs block rows (QR = G*Bs rows, 16-row
// tiles).  The waves are (query tile, key group) pairs: the key groups split
// the 32-key units of every stage that hold keys, and are merged through LDS
// when the piece ends.  Every context K/V byte is read from HBM once per step;
// a stage's K/V loads are all issued together, one stage ahead of the matrix
// work.
//
// Scores are formed transposed (S^T = K Q^T, 16x16x32 MFMA) so that each lane
// owns one query row: the online-softmax max and scale are per lane, and the
// probabilities stay in registers and feed O^T = V^T P^T directly as the B
// operand.  V is stored transposed in LDS as key pairs (one dword = two keys
// of one dimension) with an XOR swizzle of the key-pair column by the
// dimension, which keeps the transposing stores at two-way bank conflicts and
// the operand reads conflict-free.  Queries enter the bf16 products as hi/lo
// pairs (two MFMAs each), probabilities as a pair or as plain bf16 (p_lo), keys
// and values as stored.  An 8-bit cache enters the products as its integers,
// which bf16 holds exactly (|q| <= 127), and its run scales are applied in
// fp32: a score's 32-deep MFMA covers exactly one run of the key row, so each
// run's partial score is scaled by its key's run scale; on the value side the
// probabilities are scaled per key by the run scale of the output dims the
// product covers (two 16-dim slices per run).  Rounding the dequantised
// entries to bf16 instead measured 0.85% of hidden-state error at the
// Qwen3-8B shape.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dfl {

constexpr int kUnit = 32;               // keys per softmax update / PV product
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMinPieceKeys = 64;       // a workgroup's range is never cut shorter

// LDS stage of NU 32-key units.  NU = 6 (192 keys, fetched one stage ahead)
// serves chunks that fit one stage; NU = 4 (128 keys, fetched two stages
// ahead through a second register set) serves longer pieces.
template <int D, int NU, bool I8>
struct AttnLds {
  static constexpr int KS = D + 8;  // K row stride (elements)
  // V^T row length in dwords: 16 NU key pairs, padded to a power of two so the
  // column swizzle (an XOR of bits 1..4) never leaves the row
  static constexpr int VW = 16 * NU <= 64 ? 64 : 128;
  static constexpr int RS = I8 ? kUnit * NU : 1;  // 8-bit cache: run scales [run][key of the stage]
  bf16_t k[kUnit * NU * KS];
  uint32_t vt[D * VW];
  float ksc[(D / 32) * RS], vsc[(D / 32) * RS];
};

// Column of key pair kp in V^T row d.  Even, so a pair of key pairs stays
// adjacent and in order.
__device__ __forceinline__ int vt_col(int d, int kp) { return kp ^ (((d >> 3) ^ (d & 15)) << 1 & 30); }

__device__ __forceinline__ void split_out(bf16_t* hi, bf16_t* lo, size_t idx, float v) {
  const bf16_t h = f32_to_bf16_bits(v);
  hi[idx] = h;
  lo[idx] = f32_to_bf16_bits(v - bf16_bits_to_f32(h));
}

// Waves per key group (a power of two covering QT query tiles), and the key
// groups: the largest divisor of the NU units of a stage that fits the waves.
__host__ __device__ inline int attn_qtp(int QT) { return QT <= 1 ? 1 : QT <= 2 ? 2 : QT <= 4 ? 4 : 8; }
__host__ __device__ constexpr int attn_kg(int qtp, int nu) {
  return nu == 6 ? (qtp >= 8 ? 1 : qtp >= 4 ? 2 : qtp >= 2 ? 3 : 6) : (qtp >= 8 ? 1 : qtp >= 4 ? 2 : 4);
}

// Wave-wide inclusive prefix sum.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  return v;
}

// The work plan of a launch over nwg workgroups, built by one wave in LDS
// (lane l owns sequences l, l + 64, ...; all its loads are issued together;
// the caller synchronises before reading):
//   pre[b]  = sum over b' < b of L_b', L_b = T_b + Bs (a segment's keys), b = 0..B
//   wpre[b] = Hkv * sum over b' < b of n_b', n_b = max(1, floor(L_b * nwg / total))
// with total = Hkv * pre[B], and *seg_mode.  Segment mode (every segment of
// sequence b cut into n_b balanced pieces, one workgroup each, the
// workgroups of sequence b starting at wpre[b]) is taken when those pieces fit
// the grid and none is more than 5/4 of an equal share of the keys; it keeps
// every workgroup inside one segment.  Otherwise the flattened key axis is cut
// into equal ranges.  n_b is formed in fp32 (the same instructions in every
// kernel that reads the plan, so all of them agree).
__device__ __forceinline__ int range_keys(int total, int nwg);
__device__ __forceinline__ void build_plan(const int32_t* ctx_len, int B, int Bs, int Hkv, int max_ctx, int nwg,
                                           int* pre, int* wpre, int* seg_mode, int lane) {
  const int nI = (B + 63) >> 6;  // sequences per lane, at most 16
  int v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int b = lane + 64 * i;
    v[i] = i < nI && b < B ? min(max(ctx_len[b], 0), max_ctx) + Bs : 0;
  }
  int carry = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < nI) {  // wave-uniform
      const int incl = wave_incl_scan(v[i], lane) + carry;
      if (lane + 64 * i < B) pre[lane + 64 * i + 1] = incl;
      carry = __shfl(incl, 63);
    }
  }
  const int total = Hkv * carry;
  const float share = (float)nwg / (float)total;
  int wcarry = 0, longest = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i >= nI) continue;  // wave-uniform
    const int b = lane + 64 * i;
    const int n = b < B ? max(1, (int)((float)v[i] * share)) : 0;
    if (n > 0) longest = max(longest, (v[i] + n - 1) / n);
    const int incl = Hkv * wave_incl_scan(n, lane) + wcarry;
    if (b < B) wpre[b + 1] = incl;
    wcarry = __shfl(incl, 63);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) longest = max(longest, __shfl_xor(longest, off));
  if (lane == 0) {
    pre[0] = 0;
    wpre[0] = 0;
    *seg_mode = wcarry <= nwg && 4 * longest <= 5 * range_keys(total, nwg);
  }
}

// Keys per workgroup range of the flattened key axis of `total` keys.
__device__ __forceinline__ int range_keys(int total, int nwg) { return max((total + nwg - 1) / nwg, kMinPieceKeys); }

// The flattened key axis is cut in a weighted space where every segment
// carries kPieceCost extra positions in front of its keys: a workgroup's
// range then pays for each segment it starts (the query reload and the close
// of a piece cost about as much as streaming this many keys, measured), so
// workgroups that cross many short segments take fewer keys.  Weighted
// position of key k of segment (b, h): Hkv*(pre[b] + kPieceCost*b) +
// h*(L_b + kPieceCost) + kPieceCost + k.
constexpr int kPieceCost = kAttnPieceCost;
__device__ __forceinline__ int flat_weight(const int* pre, int b, int Hkv) { return Hkv * (pre[b] + kPieceCost * b); }
// Key-axis position of weighted position w (positions inside a segment's
// extra run map to the segment's first key).
__device__ __forceinline__ int flat_key_of(int w, const int* pre, int B, int Hkv) {
  int lo = 0, hi = B;  // flat_weight(lo) <= w < flat_weight(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (flat_weight(pre, mid, Hkv) <= w) lo = mid;
    else hi = mid;
  }
  const int L = pre[lo + 1] - pre[lo];
  const int off = w - flat_weight(pre, lo, Hkv);
  const int j = off / (L + kPieceCost);
  const int k = min(max(off - j * (L + kPieceCost) - kPieceCost, 0), L);
  return Hkv * pre[lo] + j * L + k;
}

// (first workgroup, pieces) of segment (b, h) under the plan in LDS: the
// workgroups of nwg whose ranges hold its keys, whose slots the merge reads.
__device__ __forceinline__ int2 segment_pieces(const int* pre, const int* wpre, int mode, int B, int Hkv, int nwg, int b,
                                               int h) {
  if (mode != 0) {
    const int np = (wpre[b + 1] - wpre[b]) / Hkv;
    return make_int2(wpre[b] + h * np, np);
  }
  const int Q = range_keys(flat_weight(pre, B, Hkv), nwg);
  const int seg_len = pre[b + 1] - pre[b];
  const int wk = flat_weight(pre, b, Hkv) + h * (seg_len + kPieceCost) + kPieceCost;  // its first key
  const int w0 = wk / Q;
  return make_int2(w0, (wk + seg_len - 1) / Q - w0 + 1);
}
// Workgroup 0 of a planned attention launch writes every segment's pieces
// for the merge (which then reads one entry instead of building the plan).
__device__ __forceinline__ void write_segment_pieces(const AttnArgs& a, const int* pre, const int* wpre, int mode) {
  if (blockIdx.x != 0) return;
  for (int s = threadIdx.x; s < a.batch * a.Hkv; s += blockDim.x)
    a.seg_info[s] = segment_pieces(pre, wpre, mode, a.batch, a.Hkv, gridDim.x, s / a.Hkv, s % a.Hkv);
}

// Largest b in [0, B) with key(b) <= x, for key nondecreasing over [0, B].
template <typename F>
__device__ __forceinline__ int upper_index(int B, int x, F key) {
  int lo = 0, hi = B;  // key(lo) <= x < key(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (key(mid) <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

// The piece a workgroup computes: segment (b, h) of length seg_len starting at
// sstart on the flattened key axis; keys [pstart, pend) of it are the
// workgroup's.
struct Piece {
  int b, h, seg_len, sstart, pstart, pend;
};

// First piece of this workgroup's range under the plan in LDS (segment mode:
// one balanced piece of one segment; else the flattened range of weighted
// keys).  False when the workgroup has no key.  g1: end of the range on the
// flattened axis.
__device__ __forceinline__ bool planned_first_piece(const AttnArgs& a, const int* pre, const int* wpre, int mode,
                                                    Piece& p, int& g1) {
  const int Hkv = a.Hkv;
  if (mode != 0) {
    const int w = blockIdx.x;
    if (w >= wpre[a.batch]) return false;
    p.b = __builtin_amdgcn_readfirstlane(upper_index(a.batch, w, [&](int i) { return wpre[i]; }));
    p.seg_len = __builtin_amdgcn_readfirstlane(pre[p.b + 1] - pre[p.b]);
    const int nb = (wpre[p.b + 1] - wpre[p.b]) / Hkv;
    const int idx = w - wpre[p.b];
    p.h = __builtin_amdgcn_readfirstlane(idx / nb);
    const int k = idx - p.h * nb;
    p.sstart = Hkv * pre[p.b] + p.h * p.seg_len;
    p.pstart = (int)((int64_t)k * p.seg_len / nb);
    p.pend = (int)((int64_t)(k + 1) * p.seg_len / nb);
    g1 = p.sstart + p.pend;
    return true;
  }
  const int wtot = flat_weight(pre, a.batch, Hkv);
  const int Q = range_keys(wtot, gridDim.x);
  const int w0 = blockIdx.x * Q;
  if (w0 >= wtot) return false;
  const int g0 = __builtin_amdgcn_readfirstlane(flat_key_of(w0, pre, a.batch, Hkv));
  g1 = __builtin_amdgcn_readfirstlane(flat_key_of(min(wtot, w0 + Q), pre, a.batch, Hkv));
  if (g0 >= g1) return false;  // the range holds no key (inside a segment's extra run)
  p.b = __builtin_amdgcn_readfirstlane(upper_index(a.batch, g0, [&](int i) { return Hkv * pre[i]; }));
  p.seg_len = __builtin_amdgcn_readfirstlane(pre[p.b + 1] - pre[p.b]);
  const int base = Hkv * pre[p.b];
  p.h = __builtin_amdgcn_readfirstlane((g0 - base) / p.seg_len);
  p.sstart = base + p.h * p.seg_len;
  p.pstart = g0 - p.sstart;
  p.pend = min(p.seg_len, g1 - p.sstart);
  return true;
}

// Next stage of a range (c: the stage's first key in segment coordinates,
// advanced by `stage` keys); at a piece end the range moves on to the next
// segment.  False when the range is done.
__device__ __forceinline__ bool next_stage(Piece& q, int& c, int stage, int g1, const int* pre, int Hkv) {
  c += stage;
  if (c < q.pend) return true;
  q.sstart += q.seg_len;
  if (q.sstart >= g1) return false;
  if (++q.h == Hkv) {
    q.h = 0;
    ++q.b;
    q.seg_len = __builtin_amdgcn_readfirstlane(pre[q.b + 1] - pre[q.b]);
  }
  q.pstart = 0;
  q.pend = min(q.seg_len, g1 - q.sstart);
  c = 0;
  return true;
}

// QTP (waves per key group, >= the query tiles) is a template parameter so
// that a wave's key units unroll completely; PLO: probabilities enter the PV
// product as a hi/lo pair (else plain bf16).
template <typename S, int D, int QTP, bool PLO, int NU>
__global__ void __launch_bounds__(kThreads) attention_kernel(const AttnArgs a) {
  constexpr int kUnits = NU;                // units per LDS stage
  constexpr int kStage = kUnit * kUnits;    // keys per LDS stage
  constexpr int PF = NU == 4 ? 2 : 1;       // stages in flight ahead of the matrix work
  constexpr int KG = attn_kg(QTP, NU);      // key groups
  constexpr int UPG = kUnits / KG;          // 32-key units per key group and stage
  static_assert(KG * QTP <= kWaves && UPG * KG == kUnits, "wave layout");
  constexpr bool I8 = std::is_same<S, int8_t>::value;  // 8-bit cache with run scales
  using Lds = AttnLds<D, NU, I8>;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  Lds& L = *reinterpret_cast<Lds*>(lds_raw);
  int* pre = reinterpret_cast<int*>(lds_raw + sizeof(Lds));  // [2][kAttnMaxBatch + 1] + 1
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.Hq / a.Hkv;
  const int QR = G * a.Bs;
  const int QT = (QR + 15) / 16;
  const int qt = wave % QTP, kg = wave / QTP;
  const bool computes = qt < QT && kg < KG;
  const int Hkv = a.Hkv, Bs = a.Bs;

  // ---- query rows of the current piece: lane's row r = 16*qt + (lane & 15)
  const int r = 16 * qt + (lane & 15);
  const bool qvalid = computes && r < QR;
  const int rr = qvalid ? r : 0;
  const int gq = rr / Bs, iq = rr - gq * Bs;
  const int HqD = a.Hq * D;
  bf16x8 qf[D / 32], qr[D / 32];  // query = qf + qr (hi/lo pair)
  auto q_load = [&](const Piece& q) {
    const size_t qoff = (size_t)(q.b * Bs + iq) * HqD + (q.h * G + gq) * D;
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
  };

  const S* kc = reinterpret_cast<const S*>(a.kc);
  const S* vc = reinterpret_cast<const S*>(a.vc);
  const size_t row = (size_t)Hkv * D;  // elements between consecutive keys
  // ---- staging through registers.  K: (key, piece) items, a piece being 8
  // dims (16 for the 8-bit cache, one 16-byte load either way).  V: (key
  // pair, piece) items in blocks of 32 key pairs; the two half-blocks of 16
  // take key pairs 16 apart (the bank pattern the V^T swizzle is built for).
  constexpr int PW = I8 && (kStage * D / 16) % kThreads == 0 ? 16 : 8;  // dims per piece
  constexpr int PIECES = D / PW;
  constexpr int KITEMS = kStage * PIECES;
  constexpr int VITEMS = (kStage / 2) * PIECES;
  constexpr int KPT = KITEMS / kThreads;
  constexpr int VPT = (VITEMS + kThreads - 1) / kThreads;
  static_assert(KITEMS % kThreads == 0 && VITEMS % 64 == 0, "stage items must fill whole waves");
  // 8-bit cache: PW integers per load (in Raw8::lo), to fp32 exactly
  auto load_piece = [&](Raw8& r, const S* src) {
    if constexpr (I8 && PW == 16) r.lo = *reinterpret_cast<const u32x4*>(src);
    else load_raw8<S>(r, src);
  };
  auto i8_to_f32 = [](const Raw8& r, float (&f)[PW]) {
#pragma unroll
    for (int w = 0; w < PW / 4; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) f[4 * w + i] = (float)((int32_t)(r.lo[w] << (24 - 8 * i)) >> 24);
  };
  // 8-bit cache: the D/32 run scales of one key row (one load per thread:
  // K rows of the stage's keys, then V rows; threads past 2 kStage repeat a
  // row so that every thread has the same loads in flight)
  using RunScales = float __attribute__((ext_vector_type(D / 32)));
  struct StageRegs {
    Raw8 k[KPT], v[VPT][2];
    RunScales sc;
  };
  const int sc_item = tid % (2 * kStage);
  const bool sc_v = sc_item >= kStage;
  const int sc_key = sc_v ? sc_item - kStage : sc_item;
  auto v_item = [&](int idx, int& kp, int& pc) {
    pc = idx % PIECES;
    const int h = (idx / PIECES) & 1, rest = idx / (2 * PIECES);
    kp = (rest & 15) + 16 * h + 32 * (rest >> 4);
  };
  // Loads are unconditional within the stage's items: a key past the piece
  // (or past the cache) re-reads the piece's last key and is zeroed at the
  // store.  The stage's base address is wave-uniform and a lane's offset is
  // min(key, lim) rows with a uniform lim, so the loads of a stage go out
  // together without branches and with little address arithmetic.
  auto stage_load = [&](StageRegs& R, const Piece& q, int c) {
    const int lim = min(a.max_ctx, q.pend) - 1 - c;  // last key of the stage that exists
    const size_t base = ((size_t)q.b * a.max_ctx + c) * row + q.h * D;
    const S* kq = kc + base;
    const S* vq = vc + base;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * kThreads;
      const int key = idx / PIECES, p8 = (idx % PIECES) * PW;
      const int off = min(key, lim) * (int)row + p8;
      load_piece(R.k[i], kq + off);
    }
    if constexpr (I8) {
      const float* sb = sc_v ? a.vs : a.ks;
      R.sc = *reinterpret_cast<const RunScales*>(sb + ((base + (size_t)min(sc_key, lim) * row) >> 5));
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * kThreads;
      if (idx >= VITEMS) continue;  // whole waves
      int kp, pc;
      v_item(idx, kp, pc);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int off = min(2 * kp + t, lim) * (int)row + PW * pc;
        load_piece(R.v[i][t], vq + off);
      }
    }
  };
  // V^T dwords are key pairs of one dimension: for bf16 storage a byte
  // permute of the two keys' dwords, for fp32 storage a conversion.  Keys past
  // the piece are zeroed (only in a piece's last stage).
  auto stage_store = [&](const StageRegs& R, const Piece& q, int c) {
    int t0 = tid;  // opaque: the store addresses are recomputed per stage, not kept live
    asm volatile("" : "+v"(t0));
    const int nvalid = q.pend - c;  // keys of the stage inside the piece
    const bool full = nvalid >= kStage;
    if constexpr (I8) {  // run scales [run][key]; a key past the piece gets 0
      if (tid < 2 * kStage) {
        float* dst = sc_v ? L.vsc : L.ksc;
        const bool ok = full || sc_key < nvalid;
#pragma unroll
        for (int rn = 0; rn < D / 32; ++rn) dst[rn * Lds::RS + sc_key] = ok ? R.sc[rn] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * kThreads;
      const int key = idx / PIECES, p8 = (idx % PIECES) * PW;
      if constexpr (I8) {
        // the integers, exact in bf16: the high half of each one's fp32 bits.
        // A key past the piece keeps its (finite) integers: its run scale is
        // 0 and its score is masked.
        float f[PW];
        i8_to_f32(R.k[i], f);
        u32x4 w[PW / 8];
#pragma unroll
        for (int j = 0; j < PW / 2; ++j)
          w[j >> 2][j & 3] = __builtin_amdgcn_perm(__float_as_uint(f[2 * j + 1]), __float_as_uint(f[2 * j]), 0x07060302u);
#pragma unroll
        for (int j = 0; j < PW / 8; ++j) *reinterpret_cast<u32x4*>(&L.k[key * Lds::KS + p8 + 8 * j]) = w[j];
      } else {
        bf16x8 v = raw_to_bf16x8<S>(R.k[i]);
        if (!full && key >= nvalid) v = bf16x8{};
        *reinterpret_cast<bf16x8*>(&L.k[key * Lds::KS + p8]) = v;
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = t0 + i * kThreads;
      if (idx >= VITEMS) continue;
      int kp, pc;
      v_item(idx, kp, pc);
      const bool ok0 = full || 2 * kp < nvalid, ok1 = full || 2 * kp + 1 < nvalid;
      if constexpr (sizeof(S) == 2) {
        u32x4 k0 = R.v[i][0].lo, k1 = R.v[i][1].lo;
        if (!ok0) k0 = u32x4{0u, 0u, 0u, 0u};
        if (!ok1) k1 = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 8 * pc + 2 * j;
          L.vt[d * Lds::VW + vt_col(d, kp)] = __builtin_amdgcn_perm(k1[j], k0[j], 0x05040100u);
          L.vt[(d + 1) * Lds::VW + vt_col(d + 1, kp)] = __builtin_amdgcn_perm(k1[j], k0[j], 0x07060302u);
        }
      } else if constexpr (I8) {
        // integers as above; a key past the piece has probability 0 and run
        // scale 0, and its integers are finite
        float v0[PW], v1[PW];
        i8_to_f32(R.v[i][0], v0);
        i8_to_f32(R.v[i][1], v1);
#pragma unroll
        for (int e = 0; e < PW; ++e) {
          const int d = PW * pc + e;
          L.vt[d * Lds::VW + vt_col(d, kp)] = __builtin_amdgcn_perm(__float_as_uint(v1[e]), __float_as_uint(v0[e]), 0x07060302u);
        }
      } else {
        float v0[8], v1[8];
        raw_to_f32x8<S>(R.v[i][0], v0);
        raw_to_f32x8<S>(R.v[i][1], v1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 8 * pc + e;
          const uint32_t lo = ok0 ? (uint32_t)f32_to_bf16_bits(v0[e]) : 0u;
          const uint32_t hi = ok1 ? (uint32_t)f32_to_bf16_bits(v1[e]) : 0u;
          L.vt[d * Lds::VW + vt_col(d, kp)] = lo | (hi << 16);
        }
      }
    }
  };

  // ---- this workgroup's piece(s)
  Piece p;
  int g1;                 // end of the workgroup's range on the flattened axis
  StageRegs R;
  bool staged = false;    // the first stage's loads are already in flight
  int* wpre = pre + kAttnMaxBatch + 1;
  int* mode = wpre + kAttnMaxBatch + 1;
  if (a.fixed_chunk > 0) {
    // fixed chunks: segment and chunk from the workgroup index; the queries
    // and the chunk's first stage (every key of it inside the cache) are
    // loaded together with the context length
    const int C = a.fixed_chunk;
    const int sg = blockIdx.x / a.fixed_pieces, k = blockIdx.x - sg * a.fixed_pieces;
    p.b = sg / Hkv;
    p.h = sg - p.b * Hkv;
    const int craw = a.ctx_len[p.b];
    p.pstart = k * C;
    p.sstart = 0;
    if (p.pstart >= a.max_ctx) return;
    Piece ps = p;
    ps.seg_len = a.max_ctx;
    ps.pend = min(p.pstart + C, a.max_ctx);
    q_load(ps);
    stage_load(R, ps, ps.pstart);
    staged = true;
    p.seg_len = min(min(max(craw, 0), a.max_ctx) + Bs, a.max_ctx);
    p.pend = min(p.pstart + C, p.seg_len);
    if (p.pstart >= p.pend) return;
    g1 = p.pend;
  } else {
    if (wave == 0) build_plan(a.ctx_len, a.batch, Bs, Hkv, a.max_ctx, gridDim.x, pre, wpre, mode, lane);
    __syncthreads();
    write_segment_pieces(a, pre, wpre, *mode);
    if (!planned_first_piece(a, pre, wpre, *mode, p, g1)) return;
  }
  int c0 = p.pstart;  // first key of the current stage, in segment coordinates
  auto advance = [&](Piece& q, int& c) -> bool { return next_stage(q, c, kStage, g1, pre, Hkv); };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) o[ds] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- one stage: for each chunk of up to three of the wave's units, the
  // scores S^T[key][q] (independent MFMA chains), one softmax update and one
  // rescale, then O^T += V^T P^T.  The LDS addresses are recomputed from an
  // opaque copy of the lane index in every stage: hoisted out of the stage loop
  // they would not fit the registers, and their spill reloads would wait for
  // the next stage's K/V loads.
  constexpr int UC = UPG < 3 ? UPG : 3;  // units per softmax update
  auto compute_units = [&](int c, int j1, int ub) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    f32x4 sc[UC][2];
#pragma unroll
    for (int uu = 0; uu < UC; ++uu) {
      const int u = ub + uu;
#pragma unroll
      for (int h = 0; h < 2; ++h) sc[uu][h] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (c + kUnit * u >= j1) continue;
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
              &L.k[(kUnit * u + 16 * h + (ln & 15)) * Lds::KS + 32 * s + 8 * (ln >> 4)]);
          if constexpr (I8) {  // one run of the key rows: scale its partial scores per key
            f32x4 t = mfma16x16x32(kf, qf[s], f32x4{0.f, 0.f, 0.f, 0.f});
            t = mfma16x16x32(kf, qr[s], t);
            const f32x4 ks4 = *reinterpret_cast<const f32x4*>(&L.ksc[s * Lds::RS + kUnit * u + 16 * h + 4 * (ln >> 4)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[uu][h][e] += t[e] * ks4[e];
          } else {
            sc[uu][h] = mfma16x16x32(kf, qf[s], sc[uu][h]);
            sc[uu][h] = mfma16x16x32(kf, qr[s], sc[uu][h]);
          }
        }
    }
    // lane holds keys c + 32*u + 16*h + 4*(lane>>4) + e for query row (lane & 15)
    float cmax = -INFINITY;
#pragma unroll
    for (int uu = 0; uu < UC; ++uu)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (c + kUnit * (ub + uu) + 16 * h + 4 * (lane >> 4) + e >= j1) sc[uu][h][e] = -INFINITY;
          cmax = fmaxf(cmax, sc[uu][h][e]);
        }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    if (m_new == -INFINITY) return;  // no valid key in these units
    const float alpha = fast_exp2(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int uu = 0; uu < UC; ++uu)
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
    // O^T[d][q] += V^T[d][keys] P^T[keys][q]; P as a hi/lo pair
#pragma unroll
    for (int uu = 0; uu < UC; ++uu) {
      const int u = ub + uu;
      if (c + kUnit * u >= j1) continue;
      const int kp0 = (kUnit / 2) * u + 2 * (ln >> 4);  // keys 32*u + 4*(lane>>4) + [0, 4)
      // the probabilities (times the keys' run scales, 8-bit cache) as the B operand
      auto p_operand = [&](const f32x4& s0, const f32x4& s1, bf16x8& ph, bf16x8& pl) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = sc[uu][0][e] * s0[e];
          p[4 + e] = sc[uu][1][e] * s1[e];
        }
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (PLO) {
            split_bf16x2(p[2 * w], p[2 * w + 1], hb[w], lb[w]);
          } else {
            typedef float f32x2_t __attribute__((ext_vector_type(2)));
            typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
            hb[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{p[2 * w], p[2 * w + 1]}, bf16x2_t));
          }
        }
        ph = __builtin_bit_cast(bf16x8, u32x4{hb[0], hb[1], hb[2], hb[3]});
        if constexpr (PLO) pl = __builtin_bit_cast(bf16x8, u32x4{lb[0], lb[1], lb[2], lb[3]});
      };
      auto pv_slice = [&](int ds, const bf16x8& ph, const bf16x8& pl) {
        const int d = 16 * ds + (ln & 15);
        const uint32_t* vrow = &L.vt[d * Lds::VW];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + vt_col(d, kp0));
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + vt_col(d, kp0 + 8));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        o[ds] = mfma16x16x32(vf, ph, o[ds]);
        if constexpr (PLO) o[ds] = mfma16x16x32(vf, pl, o[ds]);
      };
      if constexpr (I8) {
#pragma unroll
        for (int rn = 0; rn < D / 32; ++rn) {  // dims of run rn: slices 2rn, 2rn + 1
          const float* vs = &L.vsc[rn * Lds::RS + kUnit * u + 4 * (ln >> 4)];
          bf16x8 ph, pl;
          p_operand(*reinterpret_cast<const f32x4*>(vs), *reinterpret_cast<const f32x4*>(vs + 16), ph, pl);
          pv_slice(2 * rn, ph, pl);
          pv_slice(2 * rn + 1, ph, pl);
        }
      } else {
        const f32x4 one = {1.f, 1.f, 1.f, 1.f};
        bf16x8 ph, pl;
        p_operand(one, one, ph, pl);
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) pv_slice(ds, ph, pl);
      }
    }
  };
  // the stage's units that hold keys are split evenly over the key groups
  auto compute = [&](int c, int j1) {
    if (!computes) return;
    const int nu = min(kUnits, (j1 - c + kUnit - 1) / kUnit);
    const int per = (nu + KG - 1) / KG;
    const int u0 = kg * per;
    const int jg = min(j1, c + kUnit * min(nu, u0 + per));  // this group's key limit
    for (int cb = 0; cb < per; cb += UC) compute_units(c, jg, u0 + cb);
  };

  // ---- close a piece: merge the key groups of each query tile through LDS
  // (group 0 keeps the result; the records reuse the stage area, so every wave
  // must be done reading the stage), then write the output or the partial.
  // Records are [group-1][tile][d-slice][lane] 16-byte slots, so a wave's LDS
  // traffic is conflict-free 16-byte accesses.
  auto close_piece = [&](const Piece& q) {
    if constexpr (KG > 1) {
      __syncthreads();
      f32x4* mo = reinterpret_cast<f32x4*>(lds_raw);                               // [KG-1][QTP][D/16][64]
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
          const float mn = fmaxf(m_run, m2);
          if (mn == -INFINITY) continue;
          const float w1 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mn);
          const float w2 = m2 == -INFINITY ? 0.f : fast_exp2(m2 - mn);
#pragma unroll
          for (int ds = 0; ds < D / 16; ++ds) o[ds] = o[ds] * w1 + mo[(g * (D / 16) + ds) * 64 + lane] * w2;
          l_run = l_run * w1 + l2 * w2;
          m_run = mn;
        }
      }
    }
    if (computes && kg == 0) {
      // lane (q = lane & 15) holds O^T rows d = 16*ds + 4*(lane>>4) + e
      float l_tot = l_run + __shfl_xor(l_run, 16);
      l_tot += __shfl_xor(l_tot, 32);
      if (q.pstart == 0 && q.pend == q.seg_len) {  // the whole segment: final output
        if (qvalid) {
          bf16_t* out_h = reinterpret_cast<bf16_t*>(a.out_hi);
          bf16_t* out_l = reinterpret_cast<bf16_t*>(a.out_lo);
          const size_t qoff = (size_t)(q.b * Bs + iq) * HqD + (q.h * G + gq) * D;
          const float inv = 1.0f / l_tot;
#pragma unroll
          for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              split_out(out_h, out_l, qoff + 16 * ds + 4 * (lane >> 4) + e, o[ds][e] * inv);
        }
      } else if (qvalid) {
        const size_t slot = (size_t)blockIdx.x + q.b * Hkv + q.h;
        float* po = a.part_o + (slot * QR + r) * D;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) *reinterpret_cast<f32x4*>(po + 16 * ds + 4 * (lane >> 4)) = o[ds];
        if ((lane >> 4) == 0) {
          a.part_ml[(slot * QR + r) * 2 + 0] = m_run;
          a.part_ml[(slot * QR + r) * 2 + 1] = l_tot;
        }
      }
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) o[ds] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // ---- pipeline: the loads of the stage PF ahead are issued before the
  // matrix work of the current one (into the register set whose stage is
  // already in LDS), the next stage is stored to LDS after it
  struct Stage {
    Piece p;
    int c;
  };
  Stage s0{p, c0}, s1 = s0, s2;
  bool m1 = advance(s1.p, s1.c), m2 = false;
  if (PF == 2 && m1) {
    s2 = s1;
    m2 = advance(s2.p, s2.c);
  }
  StageRegs rb;
  if (!staged) {
    q_load(p);
    stage_load(R, s0.p, s0.c);
  }
  if (PF == 2 && m1) stage_load(rb, s1.p, s1.c);
  stage_store(R, s0.p, s0.c);
  __syncthreads();
  // one stage: `cur` holds the stage now in LDS (free), `nxt` the next one
  // With two stages in flight, the loads of a step go out unconditionally
  // (with no stage left to fetch, the current one is fetched again, in bounds
  // and unused) and a piece's query loads are waited for where they are
  // issued: every path then has the same loads in flight, so the waits the
  // compiler places before the stores and the matrix work count exactly the
  // loads they need.  With a varying count it waits for all loads in flight,
  // the ones of the stage ahead too.  (With one stage in flight the store
  // waits for the step's own loads anyway.)
  auto step = [&](StageRegs& cur, StageRegs& nxt) -> bool {
    if constexpr (PF == 2) {
      stage_load(cur, m2 ? s2.p : s0.p, m2 ? s2.c : s0.c);
    } else {
      if (m1) stage_load(cur, s1.p, s1.c);
    }
    compute(s0.c, s0.p.pend);
    const bool ends = !m1 || s1.p.sstart != s0.p.sstart;
    if (ends) close_piece(s0.p);
    if (!m1) return false;
    __syncthreads();
    stage_store(PF == 2 ? nxt : cur, s1.p, s1.c);
    __syncthreads();
    if (ends) {
      q_load(s1.p);
      wait_vm_all();
    }
    s0 = s1;
    if (PF == 2) {
      s1 = s2;
      m1 = m2;
      if (m2) m2 = advance(s2.p, s2.c);
    } else {
      m1 = advance(s1.p, s1.c);
    }
    return true;
  };
  if constexpr (PF == 1) {
    while (step(R, R)) {
    }
  } else {
    while (step(R, rb) && step(rb, R)) {
    }
  }
}

// ---------------------------------------------------------------- bf16 cache: LDS ring fed by LDS-DMA
// The bf16 cache takes a second form of the same piece computation, built on
// two gfx950 LDS paths:
//  * global_load_lds_dwordx4 writes a lane's 16 bytes straight into LDS at
//    the wave-uniform block address + 16 * lane, so one load instruction fills
//    one 1 KB block, in whatever order the lanes' global addresses pick.  No
//    registers hold a stage and no store instructions move it.
//  * ds_read_b64_tr_b16 reads 8 bytes per lane and transposes 16-bit elements
//    inside every group of 16 lanes: lane i of a group receives, as element e,
//    element i % 4 of the 8 bytes lane 4e + i / 4 of the group points at.
// A stage of NU 32-key units is one slot of an NS-slot ring, in MFMA fragment
// order:
//  * K: 1 KB blocks [unit][half h][s], lane l of a block holding key
//    16h + (l & 15), dims 32s + 8(l >> 4) .. +8: the A operand of S^T = K Q^T,
//    read by one ds_read_b128 at 16 * lane.
//  * V: 1 KB blocks [unit][key half kh][dim pair dp], each two 512-byte tiles
//    [16 keys][16 dims] row-major (dims 32dp + 16t + [0, 16), t = 0, 1).  The
//    transposing read of a tile at 8 * lane gives lane (G = lane >> 4,
//    j = lane & 15) the values of dim j at keys 4G + [0, 4) of the tile; the
//    two key halves make the A operand of O^T = V^T P^T with the same
//    key-to-slot map as the probabilities' B operand.
// Both reads are contiguous across the wave: conflict-free.  Loads of a stage
// are issued NS - 1 stages ahead; each wave issues the same number of them for
// every stage, so the wait for a stage is a fixed count of loads still in
// flight.  The barriers are plain s_barrier with explicit waits: a fence would
// wait for every LDS-DMA load in flight, the prefetched stages too.

// The V operands of one 32-key unit: for every 16-dim slice ds the two key
// halves' transposing reads (tile offsets 512 * ds, plus FB KB for the second
// half), all issued in one block that waits for them before it ends.  (As an
// intrinsic, the compiler puts a wait for every LDS-DMA load in flight before
// each such read.)  The outputs are early-clobber: a read in flight must not
// land in the address register of a later one.
template <int D>
__device__ __forceinline__ void read_v_unit(const unsigned char* vbase, u32x2 (&v)[D / 16][2]);
template <>
__device__ __forceinline__ void read_v_unit<128>(const unsigned char* vbase, u32x2 (&v)[8][2]) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_void_t*)vbase;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %2, %16 offset:512\n\t"
      "ds_read_b64_tr_b16 %3, %16 offset:4608\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:1024\n\t"
      "ds_read_b64_tr_b16 %5, %16 offset:5120\n\t"
      "ds_read_b64_tr_b16 %6, %16 offset:1536\n\t"
      "ds_read_b64_tr_b16 %7, %16 offset:5632\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:6144\n\t"
      "ds_read_b64_tr_b16 %10, %16 offset:2560\n\t"
      "ds_read_b64_tr_b16 %11, %16 offset:6656\n\t"
      "ds_read_b64_tr_b16 %12, %16 offset:3072\n\t"
      "ds_read_b64_tr_b16 %13, %16 offset:7168\n\t"
      "ds_read_b64_tr_b16 %14, %16 offset:3584\n\t"
      "ds_read_b64_tr_b16 %15, %16 offset:7680\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[2][0]), "=&v"(v[2][1]), "=&v"(v[3][0]),
        "=&v"(v[3][1]), "=&v"(v[4][0]), "=&v"(v[4][1]), "=&v"(v[5][0]), "=&v"(v[5][1]), "=&v"(v[6][0]), "=&v"(v[6][1]),
        "=&v"(v[7][0]), "=&v"(v[7][1])
      : "v"(a)
      : "memory");
}
template <>
__device__ __forceinline__ void read_v_unit<64>(const unsigned char* vbase, u32x2 (&v)[4][2]) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_void_t*)vbase;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:512\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:2560\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:1024\n\t"
      "ds_read_b64_tr_b16 %5, %8 offset:3072\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:1536\n\t"
      "ds_read_b64_tr_b16 %7, %8 offset:3584\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[2][0]), "=&v"(v[2][1]), "=&v"(v[3][0]),
        "=&v"(v[3][1])
      : "v"(a)
      : "memory");
}

// max / sum of v over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes of one
// MFMA column), through the gfx950 row swaps: permlane16_swap of two copies
// of v leaves v of the lane and of its xor-16 partner in the two results
// (which one is where does not matter for max and sum), permlane32_swap the
// same for the xor-32 partner.  Register to register, no LDS round trip.
__device__ __forceinline__ float col4_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col4_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, int NU, int W>
struct RingSlot {
  static constexpr int FB = D / 32;         // 1 KB blocks per (unit, half) of K and of V
  static constexpr int KBLK = NU * 2 * FB;  // K blocks of a slot
  static constexpr int BLK = 2 * KBLK;      // K then V blocks
  static constexpr int BYTES = BLK * 1024;
  static constexpr int PER_WAVE = BLK / W;  // loads per wave per stage
  static_assert(BLK % W == 0, "a stage's blocks must split evenly over the waves");
};
// key groups of a W-wave workgroup with qtp waves per group and nu units a stage
__host__ __device__ constexpr int ring_kg(int w, int qtp, int nu) { return w / qtp < nu ? w / qtp : nu; }

template <int D, int W, int QTP, bool PLO, int NU, int NS, bool QSLOT>
__global__ void __launch_bounds__(W * 64) attention_ring_kernel(const AttnArgs a) {
  using R = RingSlot<D, NU, W>;
  constexpr int kStage = kUnit * NU;
  constexpr int KG = ring_kg(W, QTP, NU);  // key groups
  constexpr int UPG = NU / KG;          // units per key group and stage
  static_assert(KG * QTP <= W && UPG * KG == NU, "wave layout");
  static_assert(NS >= 2 && NS - 2 <= 3, "ring depth");
  static_assert((KG - 1) * QTP * (D / 16) * 64 * 16 <= R::BYTES, "key-group records fit a slot");
  extern __shared__ __align__(16) unsigned char lds_raw[];
  // wave-uniform (readfirstlane): the wave's role and key ranges live in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.Hq / a.Hkv;
  const int QR = G * a.Bs;
  const int QT = (QR + 15) / 16;
  // LDS: ring [NS slots] | queries [QT tiles][hi/lo][D/32] 1 KB blocks (QSLOT:
  // none; they pass through a ring slot that holds no stage) | key-group
  // records | plan [2][batch + 1] + 1
  static_assert(!QSLOT || QTP <= 2 * NU, "the queries of QTP tiles fill at most one slot");
  unsigned char* ring = lds_raw;
  unsigned char* qarea = lds_raw + NS * R::BYTES;
  float* mml = reinterpret_cast<float*>(qarea + (QSLOT ? 0 : QT * 2 * R::FB * 1024));  // [KG-1][QTP][64][2]
  int* pre = reinterpret_cast<int*>(mml + (KG > 1 ? KG - 1 : 1) * QTP * 64 * 2);
  int* wpre = pre + a.batch + 1;
  int* mode = wpre + a.batch + 1;
  if constexpr (QSLOT) qarea = ring + (NS - 1) * R::BYTES;  // the slot the first stages leave free
  const int qt = wave % QTP, kg = wave / QTP;
  const bool computes = qt < QT && kg < KG;
  const int Hkv = a.Hkv, Bs = a.Bs;

  // ---- query rows of the current piece: lane's row r = 16*qt + (lane & 15)
  const int r = 16 * qt + (lane & 15);
  const bool qvalid = computes && r < QR;
  const int rr = qvalid ? r : 0;
  const int gq = rr / Bs, iq = rr - gq * Bs;
  const int HqD = a.Hq * D;
  // The queries of a piece reach the registers through LDS: LDS-DMA loads
  // into the query area (block (tile, hi/lo, s): lane l holds row
  // 16 tile + (l & 15), dims 32s + 8(l >> 4); rows past QR repeat the last
  // row), then one ds_read_b128 per fragment.  (A register load followed by
  // LDS-DMA loads makes the compiler wait for all of them before the
  // register is used.)
  bf16x8 qf[D / 32], qr[D / 32];  // query = qf + qr (hi/lo pair)
  auto q_issue = [&](const Piece& q) {
    const int qblk = QT * 2 * R::FB;
    // hi or lo by arithmetic (a select of the two pointers became a load of
    // the argument block at a computed offset)
    const uintptr_t qh0 = reinterpret_cast<uintptr_t>(a.q_hi), dlo = reinterpret_cast<uintptr_t>(a.q_lo) - qh0;
    for (int b = wave; b < qblk; b += W) {  // wave-uniform count
      const int t = b / (2 * R::FB), hl = (b / R::FB) & 1, s = b % R::FB;
      const int rq = min(16 * t + (lane & 15), QR - 1);
      const int g = rq / Bs, iqr = rq - g * Bs;
      const size_t off = (size_t)(q.b * Bs + iqr) * HqD + (q.h * G + g) * D + 32 * s + 8 * (lane >> 4);
      const bf16_t* src = reinterpret_cast<const bf16_t*>(qh0 + (uintptr_t)hl * dlo) + off;
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(qarea + b * 1024), 16, 0, 0);
    }
    asm volatile("" ::: "memory");
  };
  auto q_read = [&]() {
    const int t = qt < QT ? qt : 0;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      qf[s] = *reinterpret_cast<const bf16x8*>(qarea + ((t * 2 + 0) * R::FB + s) * 1024 + 16 * lane);
      qr[s] = *reinterpret_cast<const bf16x8*>(qarea + ((t * 2 + 1) * R::FB + s) * 1024 + 16 * lane);
    }
  };

  // ---- a stage's loads: this wave's blocks wave, wave + 8, ...  A key past
  // the piece (or past the cache) re-reads the stage's last existing key; its
  // score is masked and its probability is 0.  (A fixed chunk's first stages
  // are requested before the context length is known, so there such keys can
  // be any cache rows: their values are zeroed in the PV operand.)
  const bf16_t* kc = reinterpret_cast<const bf16_t*>(a.kc);
  const bf16_t* vc = reinterpret_cast<const bf16_t*>(a.vc);
  const size_t row = (size_t)Hkv * D;
  // A lane's key within a 16-key group and its byte offset within the key
  // row, for K blocks and for V blocks (fixed over the stages): a block's
  // source is then a wave-uniform base plus min(key, last) * row bytes + the
  // column, one 24-bit multiply-add per block.
  const int kkey = lane & 15, kcol = 2 * 8 * (lane >> 4);
  const int vkey = (lane & 31) >> 1, vcol = 2 * (16 * (lane >> 5) + 8 * (lane & 1));
  const unsigned rowb = 2u * (unsigned)row;
  auto issue = [&](const Piece& q, int c, int slot) {
    const int lim = min(a.max_ctx, q.pend) - 1 - c;
    const size_t base = ((size_t)q.b * a.max_ctx + c) * row + q.h * D;
    const char* kbase = reinterpret_cast<const char*>(kc + base);
    const char* vbase = reinterpret_cast<const char*>(vc + base);
    unsigned char* sl = ring + slot * R::BYTES;
#pragma unroll
    for (int i = 0; i < R::PER_WAVE; ++i) {
      const int blk = wave + W * i;
      const char* src;
      if (blk < R::KBLK) {  // K block (unit, half, s): lane -> key 16h + (lane & 15), dims 32s + 8(lane >> 4)
        const int u = blk / (2 * R::FB), h = (blk / R::FB) & 1, s = blk % R::FB;
        const int key = min(kUnit * u + 16 * h + kkey, lim);
        src = kbase + (__umul24((unsigned)key, rowb) + (unsigned)(64 * s + kcol));
      } else {  // V block (unit, kh, dp): lane -> tile lane >> 5, key 16kh + (lane & 31) / 2, 8 dims
        const int vb = blk - R::KBLK;
        const int u = vb / (2 * R::FB), kh = (vb / R::FB) & 1, dp = vb % R::FB;
        const int key = min(kUnit * u + 16 * kh + vkey, lim);
        src = vbase + (__umul24((unsigned)key, rowb) + (unsigned)(64 * dp + vcol));
      }
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(sl + blk * 1024), 16, 0, 0);
    }
    asm volatile("" ::: "memory");  // stages are issued in order (the waits count them)
  };
  // wait until at most `ahead` stages' loads of this wave are in flight
  auto wait_stage = [&](int ahead) {
    if (ahead >= 3) wait_vm<3 * R::PER_WAVE>();
    else if (ahead == 2) wait_vm<2 * R::PER_WAVE>();
    else if (ahead == 1) wait_vm<R::PER_WAVE>();
    else wait_vm<0>();
  };

  // ---- this workgroup's first piece; its queries and first stages in flight
  Piece p;
  int g1;
  Piece ip;        // the last stage issued: piece and first key
  int ic;
  int ahead = 0;   // stages issued beyond the current one
  bool more;       // the range has stages beyond the last one issued
  if (a.fixed_chunk > 0) {
    // fixed chunks: the segment and chunk follow from the workgroup index;
    // the queries and the chunk's first stages (all inside the cache) are
    // requested before the context length arrives
    const int C = a.fixed_chunk;
    const int sg = blockIdx.x / a.fixed_pieces, k = blockIdx.x - sg * a.fixed_pieces;
    p.b = sg / Hkv;
    p.h = sg - p.b * Hkv;
    // a scalar load (constant address space): no vector-memory count to wait on
    const int craw = ((const __attribute__((address_space(4))) int32_t*)a.ctx_len)[p.b];
    p.pstart = k * C;
    p.sstart = 0;
    if (p.pstart >= a.max_ctx) return;
    Piece ps = p;
    ps.seg_len = a.max_ctx;
    ps.pend = min(p.pstart + C, a.max_ctx);
    q_issue(ps);  // the queries go out before the stages
    // the first NS - 1 stages (a stage past the chunk re-reads its last one)
    int n = 0;
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) {
      const int cj = ps.pstart + kStage * j;
      if (cj < ps.pend) n = j + 1;
      issue(ps, cj < ps.pend ? cj : ps.pstart + kStage * (n - 1), j);
    }
    p.seg_len = min(min(max(craw, 0), a.max_ctx) + Bs, a.max_ctx);
    p.pend = min(p.pstart + C, p.seg_len);
    if (p.pstart >= p.pend) {
      wait_vm<0>();  // no load may still write this workgroup's LDS when it ends
      return;
    }
    g1 = p.pend;
    ip = p;
    ic = p.pstart + kStage * (n - 1);
    more = ic + kStage < p.pend;
  } else {
    if (wave == 0) build_plan(a.ctx_len, a.batch, Bs, Hkv, a.max_ctx, gridDim.x, pre, wpre, mode, lane);
    __syncthreads();
    write_segment_pieces(a, pre, wpre, *mode);
    if (!planned_first_piece(a, pre, wpre, *mode, p, g1)) return;
    q_issue(p);  // the queries go out before the stages
    // the first NS - 1 stages of the range (once the range is done, its last
    // stage is requested again)
    ip = p;
    ic = p.pstart;
    more = true;
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) {
      if (j > 0 && more) {
        Piece t = ip;
        int tc = ic;
        more = next_stage(t, tc, kStage, g1, pre, Hkv);
        if (more) {
          ip = t;
          ic = tc;
        }
      }
      issue(ip, ic, j);
    }
    if (more) {  // is there a stage after the last one issued?
      Piece t = ip;
      int tc = ic;
      more = next_stage(t, tc, kStage, g1, pre, Hkv);
    }
  }
  // NS - 1 stages were requested (some possibly repeats); the wait for the
  // first one also covers the queries, requested before it
  ahead = NS - 2;
  bool q_pending = true;  // the piece's queries are to be read from LDS at the next step
  bool q_late = false;    // ... and were requested after stages still in flight

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) o[ds] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- matrix and softmax work of a wave's units of one stage (as in the
  // register-staged form, with the operands read from the ring slot)
  constexpr int UC = UPG < 3 ? UPG : 3;  // units per softmax update
  auto compute_units = [&](const unsigned char* sl, int c, int j1, int ub) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // (c and j1 are wave-uniform: the tests below are scalar branches, and
    // the per-lane masking work stays inside them)
    const int cu = __builtin_amdgcn_readfirstlane(c), j1u = __builtin_amdgcn_readfirstlane(j1);
    f32x4 sc[UC][2];
#pragma unroll
    for (int uu = 0; uu < UC; ++uu) {
      const int u = ub + uu;
#pragma unroll
      for (int h = 0; h < 2; ++h) sc[uu][h] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (cu + kUnit * u >= j1u) continue;
      // the query's hi and lo halves accumulate into one sum (the two halves
      // of a key tile alternate, so consecutive products are independent)
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        bf16x8 kf[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          kf[h] = *reinterpret_cast<const bf16x8*>(sl + ((u * 2 + h) * R::FB + s) * 1024 + 16 * ln);
#pragma unroll
        for (int h = 0; h < 2; ++h) sc[uu][h] = mfma16x16x32(kf[h], qf[s], sc[uu][h]);
#pragma unroll
        for (int h = 0; h < 2; ++h) sc[uu][h] = mfma16x16x32(kf[h], qr[s], sc[uu][h]);
      }
    }
    // lane holds keys c + 32*u + 16*h + 4*(lane>>4) + e for query row (lane & 15)
    if (cu + kUnit * (ub + UC) > j1u) {  // keys past the piece: masked
#pragma unroll
      for (int uu = 0; uu < UC; ++uu)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + kUnit * (ub + uu) + 16 * h + 4 * (lane >> 4) + e >= j1) sc[uu][h][e] = -INFINITY;
    }
    float cmax = -INFINITY;
#pragma unroll
    for (int uu = 0; uu < UC; ++uu)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) cmax = fmaxf(cmax, sc[uu][h][e]);
    cmax = col4_max(cmax);
    const float m_new = fmaxf(m_run, cmax);
    if (m_new == -INFINITY) return;  // no valid key in these units
    const float alpha = fast_exp2(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int uu = 0; uu < UC; ++uu)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc[uu][h][e] = fast_exp2(sc[uu][h][e] - m_new);
          psum += sc[uu][h][e];
        }
    l_run = l_run * alpha + psum;
    // the output is rescaled only when some row's running max moved (alpha
    // is 1 in every other row)
    if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) o[ds] *= alpha;
    }
    m_run = m_new;
#pragma unroll
    for (int uu = 0; uu < UC; ++uu) {
      const int u = ub + uu;
      if (cu + kUnit * u >= j1u) continue;
      bf16x8 ph, pl;
      if constexpr (PLO) {
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          split_bf16x2(sc[uu][0][2 * e], sc[uu][0][2 * e + 1], hb[e], lb[e]);
          split_bf16x2(sc[uu][1][2 * e], sc[uu][1][2 * e + 1], hb[2 + e], lb[2 + e]);
        }
        ph = __builtin_bit_cast(bf16x8, u32x4{hb[0], hb[1], hb[2], hb[3]});
        pl = __builtin_bit_cast(bf16x8, u32x4{lb[0], lb[1], lb[2], lb[3]});
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ph[e] = (__bf16)sc[uu][0][e];
          ph[4 + e] = (__bf16)sc[uu][1][e];
        }
      }
      u32x2 vr[D / 16][2];
      read_v_unit<D>(sl + (R::KBLK + u * 2 * R::FB) * 1024 + 8 * ln, vr);
      if (cu + kUnit * (u + 1) > j1u) {
        // the piece ends inside this unit: keys past it hold 0.  Dword d of
        // key half kh holds keys kb + 16 kh + 2d (low half) and + 1 (high
        // half) of every dim slice, so one mask per half serves all of them.
        const int kb = cu + kUnit * u + 4 * (ln >> 4);
        u32x2 mk[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int d = 0; d < 2; ++d)
            mk[kh][d] = (kb + 16 * kh + 2 * d < j1u ? 0x0000ffffu : 0u) | (kb + 16 * kh + 2 * d + 1 < j1u ? 0xffff0000u : 0u);
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) vr[ds][kh] &= mk[kh];
      }
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{vr[ds][0][0], vr[ds][0][1], vr[ds][1][0], vr[ds][1][1]});
        o[ds] = mfma16x16x32(vf, ph, o[ds]);
        if constexpr (PLO) o[ds] = mfma16x16x32(vf, pl, o[ds]);
      }
    }
  };
  // the stage's units that hold keys are split evenly over the key groups
  auto compute = [&](const unsigned char* sl, int c, int j1) {
    if (!computes) return;
    const int nu = min(NU, (j1 - c + kUnit - 1) / kUnit);
    const int per = (nu + KG - 1) / KG;
    const int u0 = kg * per;
    const int jg = min(j1, c + kUnit * min(nu, u0 + per));
    for (int cb = 0; cb < per; cb += UC) compute_units(sl, c, jg, u0 + cb);
  };

  // ---- close a piece: the key groups of each query tile merge through the
  // slot just computed (group 0 keeps the result), then the output or the
  // partial is written
  auto close_piece = [&](const Piece& q, unsigned char* sl) {
    if constexpr (KG > 1) {
      raw_barrier();  // every wave is done reading the slot
      f32x4* mo = reinterpret_cast<f32x4*>(sl);  // [KG-1][QTP][D/16][64]
      if (computes && kg > 0) {
        const int g = (kg - 1) * QTP + qt;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) mo[(g * (D / 16) + ds) * 64 + lane] = o[ds];
        mml[(g * 64 + lane) * 2] = m_run;
        mml[(g * 64 + lane) * 2 + 1] = l_run;
      }
      wait_lgkm0();
      raw_barrier();
      if (computes && kg == 0) {
#pragma unroll
        for (int g2 = 1; g2 < KG; ++g2) {
          const int g = (g2 - 1) * QTP + qt;
          const float m2 = mml[(g * 64 + lane) * 2], l2 = mml[(g * 64 + lane) * 2 + 1];
          const float mn = fmaxf(m_run, m2);
          if (mn == -INFINITY) continue;
          const float w1 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mn);
          const float w2 = m2 == -INFINITY ? 0.f : fast_exp2(m2 - mn);
#pragma unroll
          for (int ds = 0; ds < D / 16; ++ds) o[ds] = o[ds] * w1 + mo[(g * (D / 16) + ds) * 64 + lane] * w2;
          l_run = l_run * w1 + l2 * w2;
          m_run = mn;
        }
      }
    }
    if (computes && kg == 0) {
      const float l_tot = col4_sum(l_run);
      if (q.pstart == 0 && q.pend == q.seg_len) {  // the whole segment: final output
        if (qvalid) {
          bf16_t* out_h = reinterpret_cast<bf16_t*>(a.out_hi);
          bf16_t* out_l = reinterpret_cast<bf16_t*>(a.out_lo);
          const size_t qoff = (size_t)(q.b * Bs + iq) * HqD + (q.h * G + gq) * D;
          const float inv = 1.0f / l_tot;
#pragma unroll
          for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              split_out(out_h, out_l, qoff + 16 * ds + 4 * (lane >> 4) + e, o[ds][e] * inv);
        }
      } else if (qvalid) {
        const size_t slot = (size_t)blockIdx.x + q.b * Hkv + q.h;
        float* po = a.part_o + (slot * QR + r) * D;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) *reinterpret_cast<f32x4*>(po + 16 * ds + 4 * (lane >> 4)) = o[ds];
        if ((lane >> 4) == 0) {
          a.part_ml[(slot * QR + r) * 2 + 0] = m_run;
          a.part_ml[(slot * QR + r) * 2 + 1] = l_tot;
        }
      }
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) o[ds] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // ---- the ring: stage i sits in slot i % NS; at the top of a step the
  // stage NS - 1 ahead goes into the slot the previous stage freed
  int c = p.pstart, slot = 0;
  for (;;) {
    if (q_late) wait_vm<0>();  // a new piece's queries: requested after the stages in flight
    else wait_stage(ahead);
    raw_barrier();  // the stage is in LDS for every wave; the previous slot is free
    if (q_pending) {
      q_read();
      q_pending = q_late = false;
      if constexpr (QSLOT) {  // the queries' slot is refilled below
        wait_lgkm0();
        raw_barrier();
      }
    }
    if (more) {
      more = next_stage(ip, ic, kStage, g1, pre, Hkv);
      ++ahead;
      issue(ip, ic, (slot + ahead) % NS);
      Piece t = ip;
      int tc = ic;
      more = next_stage(t, tc, kStage, g1, pre, Hkv);
    }
    unsigned char* sl = ring + slot * R::BYTES;
    compute(sl, c, p.pend);
    Piece nx = p;
    int nc = c;
    const bool has_next = next_stage(nx, nc, kStage, g1, pre, Hkv);
    const bool ends = !has_next || nx.sstart != p.sstart;
    if (ends) close_piece(p, sl);
    if (!has_next) break;
    p = nx;
    c = nc;
    slot = slot + 1 == NS ? 0 : slot + 1;
    --ahead;
    if (ends) {  // the next piece's queries, waited for at the next step
      if constexpr (QSLOT) {  // through the slot just computed (its records are read)
        raw_barrier();
        qarea = sl;
      }
      q_issue(p);
      q_pending = q_late = true;
    }
  }
  wait_vm<0>();  // no load may still write this workgroup's LDS when it ends
}

// Merge of the partial pieces of one segment (sequence, KV head).  Lanes are
// (item, group) with SG groups per item (SG from the segment's piece count);
// an item is one query row and 4 dims.  Group g takes pieces g, g+SG, ...,
// four loads of each kind issued together, and the groups are folded by a
// fixed butterfly (deterministic).  grid: (item chunks, B * Hkv), 256 threads.
template <int D>
__global__ void __launch_bounds__(256) attention_combine_kernel(const AttnArgs a) {
  const int s = blockIdx.y, b = s / a.Hkv, h = s - b * a.Hkv;
  const int tid = threadIdx.x;
  // this segment's pieces: workgroups w0 .. w0 + np - 1 (slots w + s); loads
  // go out for np_load pieces (fixed chunks: every chunk, before the context
  // length is known; the ones past the segment end are dropped after)
  int w0, np, np_load;
  if (a.fixed_chunk > 0) {
    const int craw = a.ctx_len[b];
    w0 = s * a.fixed_pieces;
    np_load = a.fixed_pieces;
    const int seg_len = min(min(max(craw, 0), a.max_ctx) + a.Bs, a.max_ctx);
    np = (seg_len + a.fixed_chunk - 1) / a.fixed_chunk;
  } else {
    const int2 si = a.seg_info[s];  // written by the attention launch from its plan
    w0 = si.x;
    np = si.y;
    np_load = np;
    if (np <= 1) return;  // written directly by the attention kernel
  }
  const int SG = np_load <= 4 ? 1 : np_load <= 16 ? 4 : 16;
  const int per = 256 / SG;  // items per chunk
  const int G = a.Hq / a.Hkv;
  const int QR = G * a.Bs;
  const int items = QR * (D / 4);
  const int g = tid % SG, il = tid / SG;
  const size_t slot0 = (size_t)w0 + s;
  for (int chunk = blockIdx.x; chunk * per < items; chunk += gridDim.x) {
    const int item = chunk * per + il;
    const bool valid = item < items;
    const int it = valid ? item : 0;
    const int r = it / (D / 4), d4 = (it - r * (D / 4)) * 4;
    float m = -INFINITY, l = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < np_load; p0 += 4 * SG) {
      float mv[4], lv[4];
      f32x4 ov[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int pc = p0 + g + SG * k;
        mv[k] = -INFINITY;
        lv[k] = 0.f;
        ov[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (pc < np_load) {
          const size_t sl = slot0 + pc;
          mv[k] = a.part_ml[(sl * QR + r) * 2];
          lv[k] = a.part_ml[(sl * QR + r) * 2 + 1];
          ov[k] = *reinterpret_cast<const f32x4*>(a.part_o + (sl * QR + r) * D + d4);
        }
      }
      if (np <= 1) return;  // fixed chunks: the segment was one chunk, written by the attention kernel
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // a chunk past the segment holds a stale slot (any values, NaN
        // included, from an earlier call): skipped, never weighted by zero
        if (p0 + g + SG * k >= np || mv[k] == -INFINITY) continue;
        const float mn = fmaxf(m, mv[k]);
        const float w1 = m == -INFINITY ? 0.f : fast_exp2(m - mn);
        const float w2 = mv[k] == -INFINITY ? 0.f : fast_exp2(mv[k] - mn);
        acc = acc * w1 + ov[k] * w2;
        l = l * w1 + lv[k] * w2;
        m = mn;
      }
    }
    for (int x = 1; x < SG; x <<= 1) {
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
    if (g != 0 || !valid) continue;
    const float inv = 1.0f / l;
    const int gq = r / a.Bs, iq = r - gq * a.Bs;
    const size_t orow = (size_t)(b * a.Bs + iq) * (a.Hq * D) + (h * G + gq) * D + d4;
    uint32_t hv[2], lv2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float v0 = acc[2 * e] * inv, v1 = acc[2 * e + 1] * inv;
      const uint32_t h0 = f32_to_bf16_bits(v0), h1 = f32_to_bf16_bits(v1);
      hv[e] = h0 | (h1 << 16);
      lv2[e] = (uint32_t)f32_to_bf16_bits(v0 - bf16_bits_to_f32(h0)) |
               ((uint32_t)f32_to_bf16_bits(v1 - bf16_bits_to_f32(h1)) << 16);
    }
    *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(a.out_hi) + orow) = u32x2{hv[0], hv[1]};
    *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(a.out_lo) + orow) = u32x2{lv2[0], lv2[1]};
  }
}

template <int D, int NU, bool I8>
static size_t attention_lds_bytes() {
  return sizeof(AttnLds<D, NU, I8>) + (size_t)(2 * (kAttnMaxBatch + 1) + 1) * sizeof(int);
}

template <typename S, int D, int NU>
static hipError_t launch_attention_nu(const AttnArgs& a, int qtp, hipStream_t stream) {
  const size_t lds = attention_lds_bytes<D, NU, std::is_same<S, int8_t>::value>();
  auto pick = [&](auto plo) {
    constexpr bool P = decltype(plo)::value;
    return qtp == 1 ? attention_kernel<S, D, 1, P, NU>
                    : qtp == 2 ? attention_kernel<S, D, 2, P, NU>
                               : qtp == 4 ? attention_kernel<S, D, 4, P, NU> : attention_kernel<S, D, 8, P, NU>;
  };
  auto k = a.p_lo ? pick(std::true_type{}) : pick(std::false_type{});
  (void)allow_dynamic_lds(reinterpret_cast<const void*>(k), lds);
  hipLaunchKernelGGL(k, dim3(a.nwg), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

// The bf16 ring, one 8-wave workgroup per compute unit.
//  * Up to four query tiles: stages of four 32-key units (two 64 KB slots at
//    D = 128, four 32 KB slots at D = 64), the queries passing through the
//    slot the first stage leaves free.
//  * More tiles: stages of two units and a query area of its own beside three
//    slots (two at the largest shapes).
// (Measured at the Qwen3-8B shapes: two 4-wave workgroups per unit, stages of
// two units in four slots, and this form all stream the 32k-context batch-4
// cache in 138-141 us per layer; the 4-wave form was 4% slower at batch 32.)
constexpr size_t kLdsBytes = 160 * 1024;

template <int D, int NU, int W>
static size_t ring_lds_bytes(int NS, bool qslot, int QT, int qtp, int batch) {
  const int kg = ring_kg(W, qtp, NU);
  return (size_t)NS * RingSlot<D, NU, W>::BYTES + (qslot ? 0 : (size_t)QT * 2 * (D / 32) * 1024) +
         (size_t)(kg > 1 ? kg - 1 : 1) * qtp * 64 * 2 * sizeof(float) + (size_t)(2 * (batch + 1) + 1) * sizeof(int);
}

template <int D, int W, int QTP, int NU, int NS, bool QSLOT>
static hipError_t launch_ring(const AttnArgs& a, hipStream_t stream) {
  const int QT = ((a.Hq / a.Hkv) * a.Bs + 15) / 16;
  const size_t lds = ring_lds_bytes<D, NU, W>(NS, QSLOT, QT, QTP, a.batch);
  if (lds > kLdsBytes) return hipErrorInvalidValue;
  auto k = a.p_lo ? attention_ring_kernel<D, W, QTP, true, NU, NS, QSLOT>
                  : attention_ring_kernel<D, W, QTP, false, NU, NS, QSLOT>;
  (void)allow_dynamic_lds(reinterpret_cast<const void*>(k), lds);
  hipLaunchKernelGGL(k, dim3(a.nwg), dim3(W * 64), lds, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_attention_ring(const AttnArgs& a, int qtp, hipStream_t stream) {
  constexpr int NSQ = D == 128 ? 2 : 4;  // slots of the four-unit ring
  if (qtp <= 4) {
    // D = 128: stages of two units in four slots (three in flight) -- against
    // four-unit stages in two slots, 32k-context batch 4 128 -> 120 us per
    // layer, equal at batch 1 and 32
    if constexpr (D == 128)
      return qtp == 1 ? launch_ring<D, 8, 1, 2, 4, true>(a, stream)
                      : qtp == 2 ? launch_ring<D, 8, 2, 2, 4, true>(a, stream) : launch_ring<D, 8, 4, 2, 4, true>(a, stream);
    return qtp == 1 ? launch_ring<D, 8, 1, 4, NSQ, true>(a, stream)
                    : qtp == 2 ? launch_ring<D, 8, 2, 4, NSQ, true>(a, stream) : launch_ring<D, 8, 4, 4, NSQ, true>(a, stream);
  }
  const int QT = ((a.Hq / a.Hkv) * a.Bs + 15) / 16;
  if (ring_lds_bytes<D, 2, 8>(4, false, QT, qtp, a.batch) <= kLdsBytes) return launch_ring<D, 8, 8, 2, 4, false>(a, stream);
  if (ring_lds_bytes<D, 2, 8>(3, false, QT, qtp, a.batch) <= kLdsBytes) return launch_ring<D, 8, 8, 2, 3, false>(a, stream);
  return launch_ring<D, 8, 8, 2, 2, false>(a, stream);
}

template <typename S, int D>
static hipError_t launch_attention_d(const AttnArgs& a, hipStream_t stream) {
  const int QR = (a.Hq / a.Hkv) * a.Bs;
  if (QR > 16 * kWaves || a.nwg <= 0 || a.batch > kAttnMaxBatch) return hipErrorInvalidValue;
  const int qtp = attn_qtp((QR + 15) / 16);
  hipError_t e;
  if constexpr (std::is_same<S, bf16_t>::value) {
    e = launch_attention_ring<D>(a, qtp, stream);
  } else {
    // register-staged form; a fixed chunk that fits one 192-key stage takes
    // the one-stage variant
    const bool one_stage = a.fixed_chunk > 0 && a.fixed_chunk <= 6 * kUnit;
    e = one_stage ? launch_attention_nu<S, D, 6>(a, qtp, stream) : launch_attention_nu<S, D, 4>(a, qtp, stream);
  }
  if (e != hipSuccess) return e;
  // merge chunks per segment: enough for the finest grouping (16 items per
  // chunk) at small batches, about 2048 workgroups in all at large ones
  const int items = QR * (D / 4);
  const int segs = a.batch * a.Hkv;
  const int gx = std::max(1, std::min((items + 15) / 16, (2048 + segs - 1) / segs));
  hipLaunchKernelGGL(attention_combine_kernel<D>, dim3(gx, segs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename S>
static hipError_t launch_attention_s(const AttnArgs& a, hipStream_t stream) {
  if (a.D == 128) return launch_attention_d<S, 128>(a, stream);
  if (a.D == 64) return launch_attention_d<S, 64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attention(int storage, const AttnArgs& a, hipStream_t stream) {
  if (a.fixed_chunk <= 0 && a.seg_info == nullptr) return hipErrorInvalidValue;  // the merge reads the plan there
  if (a.kv_int8) return launch_attention_s<int8_t>(a, stream);
  if (storage == ST_BF16) return launch_attention_s<bf16_t>(a, stream);
  return launch_attention_s<float>(a, stream);
}

}  // namespace dfl
