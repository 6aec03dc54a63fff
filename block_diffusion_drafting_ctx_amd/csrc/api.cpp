// C ABI of the drafting hot path (see include/dflash.h): argument checks,
// workspace carving, launch planning and the per-call kernel sequences.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "../../include/dflash.h"
#include "kernels.h"

using namespace dfl;

namespace {

thread_local std::string g_last_error;

dflash_status fail(dflash_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kMaxNd = 64;
constexpr int kVerifyChunk = 8192;  // vocab entries per workgroup of the verify argmax (8 loads per thread)
constexpr int kMlpHiOnlyRows = 128;  // draft rows from which the MLP products take plain bf16 inputs
constexpr bool kUseDmaGemm = true;
constexpr int kMtTargetWgs = kCUs;   // gemm_mt workgroups to aim for (one per compute unit)
// Attention workgroups: the batch's key axis is cut into this many ranges,
// one 8-wave workgroup per compute unit (the attention kernel's registers and
// LDS allow one), so every range runs in the first dispatch round.
constexpr int kAttnWgs = kCUs;
constexpr int kAttnMinChunk = 64;  // keys

// Small batches (at least two workgroups per segment) take fixed chunks: the
// cache capacity of every segment cut into as many equal chunks as the grid
// allows, so a workgroup's keys follow from its index alone.  Larger batches
// are planned on the device from the context lengths.
void attn_grid(const dflash_config& c, int batch, AttnArgs* a) {
  const int segs = batch * c.n_kv_heads;
  a->fixed_chunk = a->fixed_pieces = 0;
  a->nwg = kAttnWgs;
  if (2 * segs > kAttnWgs) return;
  const int pieces = std::max(1, std::min(kAttnWgs / segs, (c.max_ctx + kAttnMinChunk - 1) / kAttnMinChunk));
  a->fixed_pieces = pieces;
  a->fixed_chunk = (c.max_ctx + pieces - 1) / pieces;
  a->nwg = segs * pieces;
}

const char* validate(const dflash_config* c) {
  if (!c) return "null config";
  if (c->hidden <= 0 || c->hidden % 128) return "hidden must be a positive multiple of 128";
  if (c->ffn <= 0 || c->ffn % 128) return "ffn must be a positive multiple of 128";
  if (c->head_dim != 64 && c->head_dim != 128) return "head_dim must be 64 or 128";
  if (c->n_kv_heads <= 0 || c->n_q_heads <= 0 || c->n_q_heads % c->n_kv_heads) return "bad head counts";
  if ((c->n_q_heads * c->head_dim) % 128) return "n_q_heads*head_dim must be a multiple of 128";
  if (c->n_q_heads / c->n_kv_heads * c->block > 128) return "block * (n_q_heads / n_kv_heads) must be <= 128";
  if (c->n_layers <= 0 || c->n_layers > kMaxSeg / 2) return "n_layers must be in [1, 8]";
  if (c->vocab <= 0 || c->vocab % 64) return "vocab must be a positive multiple of 64";
  if (c->block < 1 || c->block > 64) return "block must be in [1, 64]";
  if (c->n_target_layers < 1 || c->n_target_layers > 8) return "n_target_layers must be in [1, 8]";
  if (c->max_batch < 1 || c->max_ctx < 1 || c->max_fuse_rows < 1) return "bad limits";
  if (c->max_batch > kAttnMaxBatch) return "max_batch must be <= 1024";
  if ((int64_t)c->n_kv_heads * c->max_batch * ((int64_t)c->max_ctx + c->block + kAttnPieceCost) >= ((int64_t)1 << 31))
    return "n_kv_heads * max_batch * (max_ctx + block + 256) must be below 2^31";
  if (c->conv_width != 0 && c->conv_width != 3) return "conv_width must be 0 or 3";
  if (c->conv_width == 3 && 16 % c->block) return "the block conv needs block to divide 16";
  if (c->dtype != DFLASH_DTYPE_F32 && c->dtype != DFLASH_DTYPE_BF16) return "unknown dtype";
  if (c->kv_dtype != DFLASH_KV_STORAGE && c->kv_dtype != DFLASH_KV_INT8) return "unknown kv_dtype";
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return "bad eps / theta";
  return nullptr;
}

// ---------------------------------------------------------------- GEMM planning
// Launch geometry of one GEMM.  gemm_as (activation stationary, split-K) for
// up to 32 rows when the activation slice fits LDS, else gemm_mt (LDS-tiled).
bool plan_gemm(int storage, int src, int out, bool lo, int M, int N, int K, GemmArgs* a, GemmLaunch* l) {
  if (M < 1 || N % 64 || K % 128) return false;
  const int ntiles = N / 16;
  const bool lo_eff = src == SRC_SPLIT ? lo : storage == ST_F32;
  *l = GemmLaunch{};
  l->src = src;
  l->out = out;
  l->lo = lo;
  a->M = M;
  a->N = N;
  a->K = K;
  const int ksl = gemm_as_ksl(M, K, lo_eff, out == OUT_ARGMAX, ntiles, kCUs);
  if (ksl > 0) {
    // one workgroup per compute unit: the k-slices share the chip, a
    // workgroup stages its activation slice once and its waves stream
    // ceil(tpw / NW) tiles each (at most 8 waves)
    const int KS = K / ksl;
    const int per_slice = std::max(1, kCUs / KS);
    const int tpw = (ntiles + per_slice - 1) / per_slice;
    const int per_wave = (tpw + 7) / 8;
    const int NW = (tpw + per_wave - 1) / per_wave;
    l->kind = GEMM_AS;
    l->MR = M <= 16 ? 1 : 2;
    l->KS = KS;
    l->grid = dim3((ntiles + tpw - 1) / tpw, KS);
    l->threads = 64 * NW;
    l->lds = std::max(gemm_as_lds(M, ksl, lo_eff), (size_t)NW * 16 * l->MR * 8);
    l->argmax_tiles = (ntiles + tpw - 1) / tpw;  // one key per workgroup and row
    a->ksl = ksl;
    a->tpw = tpw;
    return true;
  }
  // gemm_mt: BM = 64 * MF rows by BN = 32 * NF columns per workgroup; split K
  // as far as the grid stays within one dispatch round (one 8-wave workgroup
  // per compute unit): a second, partly filled round would cost a whole
  // workgroup's time, and every k-slice adds a partial-output round trip
  // (above 128 rows the LDS-DMA kernel also takes 192-row blocks where they
  // pad the rows clearly less: 544 rows run as 3 x 192 instead of 3 x 256)
  const bool dma_ok = kUseDmaGemm && storage == ST_BF16;
  const int pad3 = 192 * ((M + 191) / 192), pad4 = 256 * ((M + 255) / 256);
  const int MF = M <= 64 ? 1 : (M <= 128 ? 2 : (dma_ok && 5 * pad3 < 4 * pad4 ? 3 : 4));
  const int nbm = (M + 64 * MF - 1) / (64 * MF);
  // (every k-slice keeps an even number of 32-deep stages: the kernel's
  // pipeline takes them in pairs)
  auto split = [&](int nbn) {
    int KS = 1;
    if (out == OUT_PARTIAL)
      while (nbn * nbm * 2 * KS <= kMtTargetWgs && (K / 32) % (4 * KS) == 0 && K / (2 * KS) >= 256) KS *= 2;
    // then the largest split that still fits the round, where there are
    // several row blocks (matrix-core bound: the 544-row fusion goes from 192
    // to 240 workgroups, 137 -> 121 us; at one row block, weight streaming,
    // the extra partials cancelled the gain)
    if (out == OUT_PARTIAL && nbm >= 2)
      for (int k2 = kMtTargetWgs / (nbn * nbm); k2 > KS; --k2)
        if ((K / 32) % (2 * k2) == 0 && K / k2 >= 256) {
          KS = k2;
          break;
        }
    return KS;
  };
  // share of the compute units the grid keeps busy over its dispatch rounds
  auto fill = [&](int wgs) { return (double)wgs / (double)(((wgs + kCUs - 1) / kCUs) * kCUs); };
  int NF = MF >= 3 ? 8 : 4;
  int nbn = (N + 32 * NF - 1) / (32 * NF);
  int KS = split(nbn);
  if (MF <= 2) {
    // 64- and 128-row blocks stream weights (one workgroup per compute unit,
    // each streaming its block's weights at a bounded per-unit rate): pick the
    // block width and k-split that minimise the busiest unit's bytes --
    // dispatch rounds x (the block's weight bytes + a ramp worth ~96 KB + a
    // quarter of the activation bytes it re-reads, mostly L2 hits) + its share
    // of the split-K partials (written, then read by the finish).  (The
    // activation term: 32k-context batch-4 fusion product 75 -> 55 us, 27B
    // batch-8 Q/K/V 58 -> 54.5 us; counted at full weight it made the LM
    // head at 64 rows 17-20% slower, preferring fewer, wider blocks.)
    double best = 0;
    // (160-column blocks at 128 rows: the 27B-shaped gate/up fills 218
    // compute units instead of 182, 116 -> 112 us; not for the LM head, where
    // the cost model's pick of them was slower, 328 -> 356 us)
    for (int nf : {2, 4, 5, 6, 8}) {
      if (nf == 8 && MF == 2) continue;  // its two 64-deep stages would not fit the LDS
      if (nf == 5 && (MF != 2 || out == OUT_ARGMAX)) continue;
      const int bn = (N + 32 * nf - 1) / (32 * nf);
      for (int ks = 1; ks <= 32; ++ks) {
        if (ks > 1 && out != OUT_PARTIAL) break;
        if ((K / 128) % ks || K / ks < 256) continue;
        const double wgs = (double)bn * nbm * ks;
        const double rounds = std::ceil(wgs / kCUs);
        const double act = 64.0 * MF * (double)(K / ks) * 2.0 * (lo_eff ? 2 : 1);
        const double cost = rounds * (32.0 * nf * (double)(K / ks) * 2.0 + 96e3 + 0.25 * act) +
                            (ks > 1 ? 8.0 * ks * (double)M * N / kCUs : 0.0);
        if (best == 0 || cost < best) {
          best = cost;
          NF = nf;
          nbn = bn;
          KS = ks;
        }
      }
    }
  }
  if (MF >= 3 && out == OUT_PARTIAL) {
    // 192-column blocks when they fill the chip clearly better (gate/up at
    // 512 rows: 256 workgroups instead of 192); their wave tile reads ~11%
    // more LDS per matrix-core op
    const int nbn6 = (N + 191) / 192, KS6 = split(nbn6);
    if (fill(nbn6 * nbm * KS6) > fill(nbn * nbm * KS) + 0.1) {
      NF = 6;
      nbn = nbn6;
      KS = KS6;
    }
  }
  // 192- and 256-row blocks with bf16 operands stream their stages through
  // LDS-DMA, and so does the fusion at 64 and 128 rows (its activation rows
  // gathered from the target's hidden states by LDS-DMA: 32k-context batch-4
  // fusion 55 -> 44 us; the 64- and 128-row layer products and LM heads were
  // 5-30% slower on that kernel than on gemm_mt, also with deeper rings)
  const bool dma = dma_ok && (MF >= 3 || src == SRC_CONCAT);
  const int units = nbn * KS;
  l->kind = dma ? GEMM_DMA : GEMM_MT;
  l->MR = MF;
  l->NF = NF;
  l->KS = KS;
  l->grid = dim3(((units + 7) / 8) * 8 * nbm);
  l->threads = 512;
  l->lds = dma ? gemm_dma_lds_bytes(MF, NF, lo_eff, false) : gemm_mt_lds_bytes(MF, NF, lo_eff);
  l->argmax_tiles = nbn;
  a->nbm = nbm;
  a->nbn = nbn;
  a->KS = KS;
  a->kslice = K / KS;
  return true;
}

// Whether the draft block's activations of M rows feed LDS-DMA products, and
// so are stored in fragment blocks by the kernel that writes them (the test
// plan_gemm makes for GEMM_DMA: bf16 storage and 192- or 256-row blocks,
// M > 128).
bool act_blocked(int storage, int M) { return kUseDmaGemm && storage == ST_BF16 && M > 128; }

// gate/up of M rows (K = hidden, F = ffn, plain bf16 input) with the SiLU
// product in the LDS-DMA kernel's epilogue: 256-row blocks of 96 gate and the
// matching 96 up columns, one k-slice, so no partials and no finish kernel.
// Only where those blocks fill the chip (the split-K plan is the faster one
// below that).
bool plan_swiglu(int storage, int M, int F, int K, GemmArgs* a, GemmLaunch* l) {
  if (!act_blocked(storage, M) || F % 96 || K % 32) return false;
  const int nbm = (M + 255) / 256, nbn = F / 96;
  if (nbn * nbm < kCUs) return false;
  *l = GemmLaunch{};
  l->kind = GEMM_DMA;
  l->src = SRC_SPLIT;
  l->out = OUT_SWIGLU;
  l->lo = 0;
  l->MR = 4;
  l->NF = 6;
  l->KS = 1;
  l->grid = dim3(((nbn + 7) / 8) * 8 * nbm);
  l->threads = 512;
  l->lds = gemm_dma_lds_bytes(4, 6, false, true);
  a->M = M;
  a->N = 2 * F;
  a->K = K;
  a->nbm = nbm;
  a->nbn = nbn;
  a->KS = 1;
  a->kslice = K;
  return true;
}

// Floats of partial tiles the planner needs for a product of this shape.
size_t partial_floats(int storage, int src, bool lo, int Mmax, int N, int K) {
  size_t best = 0;
  for (int M = 1; M <= Mmax; ++M) {
    GemmArgs a{};
    GemmLaunch l{};
    if (plan_gemm(storage, src, OUT_PARTIAL, lo, M, N, K, &a, &l)) best = std::max(best, (size_t)l.KS * M * N);
  }
  return best;
}

struct WsLayout {
  size_t err, stats;
  size_t x, ssq, rinv, y, xs_hi, xs_lo, q_hi, q_lo, kb, vb, o_hi, o_lo, act_hi, act_lo, part, lm_best, ver_best,
      part_o, part_ml, seg, rope;
  // tiled bf16 copies of the projection matrices, one per product
  size_t wt_fc, wt_kv, wt_lm, wt_qkv[kMaxSeg / 2], wt_o[kMaxSeg / 2], wt_gu[kMaxSeg / 2], wt_down[kMaxSeg / 2];
  size_t total;
  int md, mf, mmax, ssq_parts, ver_chunks, rope_rows;
};

WsLayout layout(const dflash_config& c) {
  WsLayout L{};
  const int st = c.dtype == DFLASH_DTYPE_BF16 ? ST_BF16 : ST_F32;
  const size_t H = c.hidden, D = c.head_dim, F = c.ffn;
  const int Nq = c.n_q_heads * c.head_dim, Nk = c.n_kv_heads * c.head_dim;
  L.md = c.max_batch * c.block;
  L.mf = c.max_batch * c.max_fuse_rows;
  L.mmax = std::max(L.md, L.mf);
  L.ssq_parts = c.hidden / 16;
  // attention piece slots: workgroup + segment index of every piece
  const size_t attn_slots = (size_t)kAttnWgs + (size_t)c.max_batch * c.n_kv_heads;
  const size_t QR = (size_t)(c.n_q_heads / c.n_kv_heads) * c.block;
  size_t parts = 0;
  parts = std::max(parts, partial_floats(st, SRC_CONCAT, false, L.mf, c.hidden, c.hidden * c.n_target_layers));
  parts = std::max(parts, partial_floats(st, SRC_SPLIT, false, L.mf, 2 * c.n_layers * Nk, c.hidden));
  parts = std::max(parts, partial_floats(st, SRC_SPLIT, true, L.md, c.hidden, Nq));
  for (bool lo : {true, false}) {  // the Q/K/V and MLP products take hi/lo or plain activations
    parts = std::max(parts, partial_floats(st, SRC_SPLIT, lo, L.md, Nq + 2 * Nk, c.hidden));
    parts = std::max(parts, partial_floats(st, SRC_SPLIT, lo, L.md, 2 * c.ffn, c.hidden));
    parts = std::max(parts, partial_floats(st, SRC_SPLIT, lo, L.md, c.hidden, c.ffn));
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.err = take(16);
  L.stats = take(3 * 8);
  L.x = take((size_t)L.md * H * 4);
  L.ssq = take((size_t)L.ssq_parts * L.mmax * 4);
  L.rinv = take((size_t)L.mmax * 4);
  L.y = take((size_t)L.mf * H * 4);
  // (whole 16-row groups: the fragment-block layout stores them)
  L.xs_hi = take((size_t)((L.mmax + 15) / 16 * 16) * H * 2);
  L.xs_lo = take((size_t)((L.mmax + 15) / 16 * 16) * H * 2);
  L.q_hi = take((size_t)L.md * Nq * 2);
  L.q_lo = take((size_t)L.md * Nq * 2);
  L.o_hi = take((size_t)L.md * Nq * 2);
  L.o_lo = take((size_t)L.md * Nq * 2);
  L.act_hi = take((size_t)L.md * F * 2);
  L.act_lo = take((size_t)L.md * F * 2);
  L.part = take(parts * 4);
  L.lm_best = take((size_t)(c.vocab / 16) * L.md * 8);
  L.ver_chunks = (c.vocab + kVerifyChunk - 1) / kVerifyChunk;
  L.ver_best = take((size_t)c.max_batch * (kMaxNd + 1) * L.ver_chunks * 8);
  L.part_o = take(attn_slots * QR * D * 4);
  L.part_ml = take(attn_slots * QR * 2 * 4);
  L.seg = take((size_t)c.max_batch * c.n_kv_heads * 8);
  // RoPE positions reach max_ctx + rows per sequence - 1 (block rows, or fused rows)
  L.rope_rows = c.max_ctx + std::max(c.block, c.max_fuse_rows);
  L.rope = take((size_t)L.rope_rows * (D / 2) * 8);
  L.wt_fc = take(H * H * c.n_target_layers * 2);
  L.wt_kv = take((size_t)2 * c.n_layers * Nk * H * 2);
  L.wt_lm = take((size_t)c.vocab * H * 2);
  for (int l = 0; l < c.n_layers; ++l) {
    L.wt_qkv[l] = take((size_t)(Nq + 2 * Nk) * H * 2);
    L.wt_o[l] = take(H * Nq * 2);
    L.wt_gu[l] = take(2 * F * H * 2);
    L.wt_down[l] = take(H * F * 2);
  }
  L.total = off;
  return L;
}

// Bytes of one layer's K (or V) cache and, for the 8-bit format, the byte
// offset of its run scales.
size_t kv_values_bytes(const dflash_config& c) {
  const size_t n = (size_t)c.max_batch * c.max_ctx * c.n_kv_heads * c.head_dim;
  if (c.kv_dtype == DFLASH_KV_INT8) return n;
  return n * (c.dtype == DFLASH_DTYPE_BF16 ? 2 : 4);
}
size_t kv_layer_bytes(const dflash_config& c) {
  if (c.kv_dtype != DFLASH_KV_INT8) return kv_values_bytes(c);
  const size_t n = (size_t)c.max_batch * c.max_ctx * c.n_kv_heads * c.head_dim;
  return align256(n) + n / 32 * 4;
}

struct EventPool {
  bool enabled = false;
  std::vector<hipEvent_t> begin, end;
  size_t used = 0;
};

}  // namespace

struct dflash_ctx {
  dflash_config cfg;
  WsLayout L;
  char* ws;
  const void* embed;
  const void* w_fc;
  const void* g_fc;
  const void* g_final;
  const void* w_lm;
  std::vector<const void*> w_q, w_k, w_v, w_o, w_gate, w_up, w_down, g_in, g_post, conv;
  std::vector<void*> kv_k, kv_v;
  std::vector<float*> kv_ks, kv_vs;  // run scales of an 8-bit cache (else null)
  int32_t* ctx_len;
  EventPool timing[DFLASH_N_STAGES];

  template <typename T>
  T* at(size_t off) const {
    return reinterpret_cast<T*>(ws + off);
  }
  int storage() const { return cfg.dtype == DFLASH_DTYPE_BF16 ? ST_BF16 : ST_F32; }
};

namespace {

struct StageScope {
  dflash_ctx* c;
  int stage;
  hipStream_t s;
  size_t slot = (size_t)-1;
  // Stage events are host-timed records; under stream capture (where a plain
  // record would only be a dependency marker) nothing is recorded.
  StageScope(dflash_ctx* c_, int stage_, hipStream_t s_) : c(c_), stage(stage_), s(s_) {
    EventPool& p = c->timing[stage];
    if (p.enabled && p.used < p.begin.size()) {
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
      slot = p.used++;
      (void)hipEventRecord(p.begin[slot], s);
    }
  }
  ~StageScope() {
    if (slot != (size_t)-1) (void)hipEventRecord(c->timing[stage].end[slot], s);
  }
};

dflash_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DFLASH_OK;
  return fail(DFLASH_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Tiled copies of every projection matrix (the products read only these):
// the segments of a product are laid out tile after tile in its N order.
dflash_status tile_weights(dflash_ctx* c, hipStream_t s) {
  const dflash_config& cf = c->cfg;
  const WsLayout& L = c->L;
  const int H = cf.hidden, F = cf.ffn, Nq = cf.n_q_heads * cf.head_dim, Nk = cf.n_kv_heads * cf.head_dim;
  const int st = c->storage();
  hipError_t e = hipSuccess;
  auto tile = [&](const void* src, int rows, int K, size_t dst, int row0) {
    if (e == hipSuccess) e = launch_tile_weights(st, src, rows, K, c->ws + dst, row0 / 16, s);
  };
  tile(c->w_fc, H, H * cf.n_target_layers, L.wt_fc, 0);
  tile(c->w_lm, cf.vocab, H, L.wt_lm, 0);
  for (int l = 0; l < cf.n_layers; ++l) {
    tile(c->w_k[l], Nk, H, L.wt_kv, 2 * l * Nk);  // context K^l, V^l: segments 2l, 2l + 1
    tile(c->w_v[l], Nk, H, L.wt_kv, (2 * l + 1) * Nk);
    tile(c->w_q[l], Nq, H, L.wt_qkv[l], 0);
    tile(c->w_k[l], Nk, H, L.wt_qkv[l], Nq);
    tile(c->w_v[l], Nk, H, L.wt_qkv[l], Nq + Nk);
    tile(c->w_o[l], H, Nq, L.wt_o[l], 0);
    tile(c->w_gate[l], F, H, L.wt_gu[l], 0);
    tile(c->w_up[l], F, H, L.wt_gu[l], F);
    tile(c->w_down[l], H, F, L.wt_down[l], 0);
  }
  return hip_status(e, "weight tiling");
}

// Main kernel of one product into the partial-tile buffer, then its finish kernel.
dflash_status gemm_partial(dflash_ctx* c, GemmArgs& a, int src, bool lo, int M, int N, int K, GemmLaunch* l,
                           hipStream_t s) {
  if (!plan_gemm(c->storage(), src, OUT_PARTIAL, lo, M, N, K, &a, l))
    return fail(DFLASH_EUNSUPPORTED, "no GEMM launch plan for M=" + std::to_string(M) + " N=" + std::to_string(N) +
                                         " K=" + std::to_string(K));
  a.part = c->at<float>(c->L.part);
  return hip_status(launch_gemm(c->storage(), a, *l, s), "gemm launch");
}

dflash_status finish(dflash_ctx* c, FinishKind kind, FinishArgs& f, const GemmLaunch& l, int M, int N,
                     hipStream_t s) {
  f.part = c->at<float>(c->L.part);
  f.KS = l.KS;
  f.ntiles = N / 16;
  f.M = M;
  f.N = N;
  return hip_status(launch_finish(c->storage(), kind, f, s), "finish launch");
}

}  // namespace

extern "C" {

const char* dflash_last_error(void) { return g_last_error.c_str(); }

const char* dflash_version(void) { return "dflash-mi355x 0.2 (gfx950)"; }

size_t dflash_workspace_bytes(const dflash_config* cfg) {
  if (validate(cfg)) return 0;
  return layout(*cfg).total;
}

size_t dflash_kv_layer_bytes(const dflash_config* cfg) {
  if (validate(cfg)) return 0;
  return kv_layer_bytes(*cfg);
}

dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* w, void* const* kv_k, void* const* kv_v,
                            int32_t* ctx_len, void* workspace, size_t workspace_bytes, dflash_ctx** out) {
  g_last_error.clear();
  if (!out) return fail(DFLASH_EINVAL, "null output handle");
  *out = nullptr;
  if (const char* why = validate(cfg)) return fail(DFLASH_EUNSUPPORTED, why);
  if (!w || !kv_k || !kv_v || !ctx_len || !workspace) return fail(DFLASH_EINVAL, "null argument");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(DFLASH_EINVAL, "workspace must be 256-byte aligned");
  const WsLayout L = layout(*cfg);
  if (workspace_bytes < L.total) return fail(DFLASH_EINVAL, "workspace too small");
  if (!w->embed || !w->w_fc || !w->g_fc || !w->g_final || !w->w_lm) return fail(DFLASH_EINVAL, "null weight");
  const int nl = cfg->n_layers;
  const void* const* per[] = {w->w_q, w->w_k, w->w_v, w->w_o, w->w_gate, w->w_up, w->w_down, w->g_in, w->g_post};
  for (auto arr : per) {
    if (!arr) return fail(DFLASH_EINVAL, "null per-layer weight array");
    for (int l = 0; l < nl; ++l)
      if (!arr[l]) return fail(DFLASH_EINVAL, "null per-layer weight");
  }
  if (cfg->conv_width) {
    if (!w->conv) return fail(DFLASH_EINVAL, "conv_width=3 needs conv taps");
    for (int l = 0; l < nl; ++l)
      if (!w->conv[l]) return fail(DFLASH_EINVAL, "null conv taps");
  }
  for (int l = 0; l < nl; ++l) {
    if (!kv_k[l] || !kv_v[l]) return fail(DFLASH_EINVAL, "null KV cache pointer");
    if (reinterpret_cast<uintptr_t>(kv_k[l]) % 256 || reinterpret_cast<uintptr_t>(kv_v[l]) % 256)
      return fail(DFLASH_EINVAL, "KV cache buffers must be 256-byte aligned");
  }

  dflash_ctx* c = new (std::nothrow) dflash_ctx();
  if (!c) return fail(DFLASH_EINVAL, "out of host memory");
  c->cfg = *cfg;
  c->L = L;
  c->ws = static_cast<char*>(workspace);
  c->embed = w->embed;
  c->w_fc = w->w_fc;
  c->g_fc = w->g_fc;
  c->g_final = w->g_final;
  c->w_lm = w->w_lm;
  c->w_q.assign(w->w_q, w->w_q + nl);
  c->w_k.assign(w->w_k, w->w_k + nl);
  c->w_v.assign(w->w_v, w->w_v + nl);
  c->w_o.assign(w->w_o, w->w_o + nl);
  c->w_gate.assign(w->w_gate, w->w_gate + nl);
  c->w_up.assign(w->w_up, w->w_up + nl);
  c->w_down.assign(w->w_down, w->w_down + nl);
  c->g_in.assign(w->g_in, w->g_in + nl);
  c->g_post.assign(w->g_post, w->g_post + nl);
  c->conv.assign(nl, nullptr);
  if (cfg->conv_width)
    for (int l = 0; l < nl; ++l) c->conv[l] = w->conv[l];
  c->kv_k.assign(kv_k, kv_k + nl);
  c->kv_v.assign(kv_v, kv_v + nl);
  c->kv_ks.assign(nl, nullptr);
  c->kv_vs.assign(nl, nullptr);
  if (cfg->kv_dtype == DFLASH_KV_INT8) {
    const size_t off = align256(kv_values_bytes(*cfg));
    for (int l = 0; l < nl; ++l) {
      c->kv_ks[l] = reinterpret_cast<float*>(static_cast<char*>(kv_k[l]) + off);
      c->kv_vs[l] = reinterpret_cast<float*>(static_cast<char*>(kv_v[l]) + off);
    }
  }
  c->ctx_len = ctx_len;
  hipError_t e = hipMemset(workspace, 0, L.total);
  if (e == hipSuccess)
    e = launch_rope_table(c->at<float2>(L.rope), L.rope_rows, cfg->head_dim, cfg->rope_theta, nullptr);
  if (e == hipSuccess) {
    if (const dflash_status ts = tile_weights(c, nullptr)) {
      delete c;
      return ts;
    }
    e = hipStreamSynchronize(nullptr);  // the clear, the table and the tiled copy ran on the null stream
  }
  if (e != hipSuccess) {
    delete c;
    return hip_status(e, "workspace clear");
  }
  *out = c;
  return DFLASH_OK;
}

dflash_status dflash_reload_weights(dflash_ctx* c, void* stream) {
  g_last_error.clear();
  if (!c) return fail(DFLASH_EINVAL, "null context");
  return tile_weights(c, static_cast<hipStream_t>(stream));
}

dflash_status dflash_fuse_ctx(dflash_ctx* c, int32_t batch, const void* const* hidden, int32_t t_new,
                              int32_t commit, float* feat_dbg, void* stream) {
  g_last_error.clear();
  if (!c) return fail(DFLASH_EINVAL, "null context");
  const dflash_config& cf = c->cfg;
  if (batch < 0 || batch > cf.max_batch) return fail(DFLASH_EINVAL, "batch out of range");
  if (t_new < 0 || t_new > cf.max_fuse_rows) return fail(DFLASH_EINVAL, "t_new out of range");
  if (batch == 0 || t_new == 0) return DFLASH_OK;
  if (!hidden) return fail(DFLASH_EINVAL, "null hidden array");
  for (int j = 0; j < cf.n_target_layers; ++j)
    if (!hidden[j]) return fail(DFLASH_EINVAL, "null hidden-state pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int M = batch * t_new, H = cf.hidden, D = cf.head_dim;
  const WsLayout& L = c->L;
  dflash_status st;
  {  // Y = concat(h) . W_fc^T; hi/lo of Y * g_fc; row sums of squares
    StageScope sc(c, DFLASH_STAGE_FUSE_FC, s);
    GemmArgs a{};
    GemmLaunch l{};
    a.wt = c->at<void>(L.wt_fc);
    for (int j = 0; j < cf.n_target_layers; ++j) a.src[j] = hidden[j];
    a.n_src = cf.n_target_layers;
    a.src_width = H;
    if ((st = gemm_partial(c, a, SRC_CONCAT, false, M, H, H * cf.n_target_layers, &l, s))) return st;
    FinishArgs f{};
    f.out_f32 = c->at<float>(L.y);
    f.gnext = c->g_fc;
    f.out_hi = c->at<void>(L.xs_hi);
    f.out_lo = c->at<void>(L.xs_lo);
    f.ssq_out = c->at<float>(L.ssq);
    f.ld_ssq = L.mmax;
    f.block = t_new;
    if ((st = finish(c, FIN_ROWTILE, f, l, M, H, s))) return st;
  }
  int nkv = 0;
  {  // c = RMSNorm(Y) g_fc;  [K^l ; V^l] = c . [W_k^l ; W_v^l]^T for all layers, RoPE, append
    StageScope sc(c, DFLASH_STAGE_CTX_KV, s);
    GemmArgs a{};
    GemmLaunch l{};
    FinishArgs f{};
    a.wt = c->at<void>(L.wt_kv);
    f.kv_int8 = cf.kv_dtype == DFLASH_KV_INT8;
    for (int l2 = 0; l2 < cf.n_layers; ++l2) {
      for (int kv = 0; kv < 2; ++kv) {
        f.kv_cache[2 * l2 + kv] = kv ? c->kv_v[l2] : c->kv_k[l2];
        f.kv_scale[2 * l2 + kv] = kv ? c->kv_vs[l2] : c->kv_ks[l2];
        nkv += cf.n_kv_heads * D;
      }
    }
    a.a_hi = c->at<void>(L.xs_hi);
    a.lda = H;
    a.ssq_in = c->at<float>(L.ssq);
    a.ssq_nparts = H / 16;
    a.ld_ssq = L.mmax;
    a.eps = cf.rms_eps;
    a.rinv_out = c->at<float>(L.rinv);
    // hi only: the context K/V are storage-rounded anyway
    if ((st = gemm_partial(c, a, SRC_SPLIT, false, M, nkv, H, &l, s))) return st;
    f.rinv = c->at<float>(L.rinv);
    f.rope = c->at<float2>(L.rope);
    f.block = t_new;
    f.ctx_len = c->ctx_len;
    f.max_ctx = cf.max_ctx;
    f.head_dim = D;
    f.n_q_heads = cf.n_q_heads;
    f.n_kv_heads = cf.n_kv_heads;
    f.err = c->at<uint32_t>(L.err);
    if ((st = finish(c, FIN_KV, f, l, M, nkv, s))) return st;
  }
  if (feat_dbg) {
    if ((st = hip_status(launch_feature_dbg(c->storage(), c->at<float>(L.y), c->at<float>(L.ssq), H / 16, L.mmax,
                                            c->g_fc, cf.rms_eps, M, H, feat_dbg, s),
                         "feature debug")))
      return st;
  }
  if (commit) return hip_status(launch_commit(c->ctx_len, batch, t_new, cf.max_ctx, s), "commit");
  return DFLASH_OK;
}

dflash_status dflash_verify(dflash_ctx* c, int32_t batch, const float* logits, const int32_t* draft_ids,
                            int32_t draft_stride, int32_t n_d, int32_t* n_accept, int32_t* bonus,
                            int32_t* out_tokens, void* stream) {
  g_last_error.clear();
  if (!c) return fail(DFLASH_EINVAL, "null context");
  const dflash_config& cf = c->cfg;
  if (batch < 0 || batch > cf.max_batch) return fail(DFLASH_EINVAL, "batch out of range");
  if (n_d < 0 || n_d > kMaxNd) return fail(DFLASH_EINVAL, "n_d out of range [0, 64]");
  if (batch == 0) return DFLASH_OK;
  if (!logits || !n_accept || !bonus || !out_tokens || (n_d > 0 && !draft_ids))
    return fail(DFLASH_EINVAL, "null argument");
  if (n_d > 0 && draft_stride < n_d) return fail(DFLASH_EINVAL, "draft_stride < n_d");
  VerifyArgs a{};
  a.logits = logits;
  a.draft = draft_ids;
  a.draft_stride = draft_stride;
  a.n_d = n_d;
  a.batch = batch;
  a.V = cf.vocab;
  a.max_ctx = cf.max_ctx;
  a.chunk = kVerifyChunk;
  a.nchunks = c->L.ver_chunks;
  a.part = c->at<uint64_t>(c->L.ver_best);
  a.n_accept = n_accept;
  a.bonus = bonus;
  a.out_tokens = out_tokens;
  a.ctx_len = c->ctx_len;
  a.stats = c->at<unsigned long long>(c->L.stats);
  a.err = c->at<uint32_t>(c->L.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  StageScope sc(c, DFLASH_STAGE_VERIFY, s);
  return hip_status(launch_verify(a, s), "verify launch");
}

dflash_status dflash_verify_static(int32_t batch, int32_t vocab, const float* logits, const int32_t* draft_ids,
                                   int32_t draft_stride, int32_t n_d, int32_t* ctx_len, int32_t max_ctx,
                                   int32_t* n_accept, int32_t* bonus, int32_t* out_tokens, uint64_t* stats,
                                   uint32_t* error_word, void* stream) {
  g_last_error.clear();
  if (batch < 0) return fail(DFLASH_EINVAL, "batch out of range");
  if (n_d < 0 || n_d > kMaxNd) return fail(DFLASH_EINVAL, "n_d out of range [0, 64]");
  if (vocab <= 0 || vocab % 64) return fail(DFLASH_EINVAL, "vocab must be a positive multiple of 64");
  if (max_ctx < 1) return fail(DFLASH_EINVAL, "max_ctx must be positive");
  const int nchunks = (vocab + kVerifyChunk - 1) / kVerifyChunk;
  const size_t keys = (size_t)batch * (size_t)(n_d + 1) * (size_t)nchunks;
  if (keys > kStaticVerifyKeys)
    return fail(DFLASH_EINVAL, "batch * (n_d + 1) * ceil(vocab / 8192) = " + std::to_string(keys) +
                                   " exceeds the static scratch (" + std::to_string(kStaticVerifyKeys) + " keys)");
  if (batch == 0) return DFLASH_OK;
  if (!logits || !ctx_len || !n_accept || !bonus || !out_tokens || (n_d > 0 && !draft_ids))
    return fail(DFLASH_EINVAL, "null argument");
  if (reinterpret_cast<uintptr_t>(logits) % 16) return fail(DFLASH_EINVAL, "target_logits must be 16-byte aligned");
  if (n_d > 0 && draft_stride < n_d) return fail(DFLASH_EINVAL, "draft_stride < n_d");
  uint64_t* keys_dev = nullptr;
  if (dflash_status st = hip_status(static_verify_scratch(&keys_dev), "static scratch lookup")) return st;
  VerifyArgs a{};
  a.logits = logits;
  a.draft = draft_ids;
  a.draft_stride = draft_stride;
  a.n_d = n_d;
  a.batch = batch;
  a.V = vocab;
  a.max_ctx = max_ctx;
  a.chunk = kVerifyChunk;
  a.nchunks = nchunks;
  a.part = keys_dev;
  a.n_accept = n_accept;
  a.bonus = bonus;
  a.out_tokens = out_tokens;
  a.ctx_len = ctx_len;
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  a.err = error_word;
  return hip_status(launch_verify(a, static_cast<hipStream_t>(stream)), "verify launch");
}

dflash_status dflash_verify_sample(dflash_ctx* c, int32_t batch, const float* logits, const int32_t* draft_ids,
                                   int32_t draft_stride, int32_t n_d, float temperature, const float* uniforms,
                                   int32_t* n_accept, int32_t* bonus, int32_t* out_tokens, void* stream) {
  g_last_error.clear();
  if (!c) return fail(DFLASH_EINVAL, "null context");
  const dflash_config& cf = c->cfg;
  if (batch < 0 || batch > cf.max_batch) return fail(DFLASH_EINVAL, "batch out of range");
  if (n_d < 0 || n_d > kMaxNd) return fail(DFLASH_EINVAL, "n_d out of range [0, 64]");
  // 1/T must be finite too: a subnormal T would scale every logit to +-inf
  if (!(temperature > 0.f) || !(temperature < 1e30f) || !std::isfinite(1.0f / temperature))
    return fail(DFLASH_EINVAL, "temperature must be finite and > 0, with a finite reciprocal");
  if (batch == 0) return DFLASH_OK;
  if (!logits || !uniforms || !n_accept || !bonus || !out_tokens || (n_d > 0 && !draft_ids))
    return fail(DFLASH_EINVAL, "null argument");
  if (n_d > 0 && draft_stride < n_d) return fail(DFLASH_EINVAL, "draft_stride < n_d");
  VerifyArgs a{};
  a.logits = logits;
  a.draft = draft_ids;
  a.draft_stride = draft_stride;
  a.n_d = n_d;
  a.batch = batch;
  a.V = cf.vocab;
  a.max_ctx = cf.max_ctx;
  a.chunk = kVerifyChunk;
  a.nchunks = c->L.ver_chunks;
  a.part = c->at<uint64_t>(c->L.ver_best);
  a.n_accept = n_accept;
  a.bonus = bonus;
  a.out_tokens = out_tokens;
  a.ctx_len = c->ctx_len;
  a.stats = c->at<unsigned long long>(c->L.stats);
  a.err = c->at<uint32_t>(c->L.err);
  a.inv_temp = 1.0f / temperature;
  a.uniforms = uniforms;
  hipStream_t s = static_cast<hipStream_t>(stream);
  StageScope sc(c, DFLASH_STAGE_VERIFY, s);
  return hip_status(launch_verify_sample(a, s), "verify launch");
}

dflash_status dflash_draft_block(dflash_ctx* c, int32_t batch, const int32_t* block_ids, int32_t* draft_ids,
                                 float* logits_dbg, float* hidden_dbg, void* stream) {
  g_last_error.clear();
  if (!c) return fail(DFLASH_EINVAL, "null context");
  const dflash_config& cf = c->cfg;
  if (batch < 0 || batch > cf.max_batch) return fail(DFLASH_EINVAL, "batch out of range");
  if (batch == 0) return DFLASH_OK;
  if (!block_ids || !draft_ids) return fail(DFLASH_EINVAL, "null argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const WsLayout& L = c->L;
  const int M = batch * cf.block, H = cf.hidden, D = cf.head_dim, F = cf.ffn;
  const int Nq = cf.n_q_heads * D, Nk = cf.n_kv_heads * D;
  float* x = c->at<float>(L.x);
  float* ssq = c->at<float>(L.ssq);
  void* xs_hi = c->at<void>(L.xs_hi);
  void* xs_lo = c->at<void>(L.xs_lo);
  dflash_status st;
  {
    StageScope sc(c, DFLASH_STAGE_EMBED, s);
    // (the lo half only where the first Q/K/V product takes the pair)
    st = hip_status(launch_embed(c->storage(), c->embed, c->g_in[0], block_ids, M, H, cf.vocab, x, xs_hi,
                                 c->storage() == ST_F32 ? xs_lo : nullptr, act_blocked(c->storage(), M), ssq,
                                 L.mmax, c->at<uint32_t>(L.err), s),
                    "embed launch");
    if (st) return st;
  }
  int ssq_parts = H / 128;  // the embedding's partial sums of squares per row
  float* rinv = c->at<float>(L.rinv);
  // RMSNorm of the product's activation rows: its main kernel turns the
  // partial sums of squares into row scales for the finish kernel
  auto norm = [&](GemmArgs& a, FinishArgs& f) {
    a.ssq_in = ssq;
    a.ssq_nparts = ssq_parts;
    a.ld_ssq = L.mmax;
    a.eps = cf.rms_eps;
    a.rinv_out = rinv;
    f.rinv = rinv;
  };
  // The MLP inputs (normalised residual into gate/up, SiLU product into down)
  // and the attention probabilities enter their products as a hi/lo pair
  // while the products stream weights or wait on memory (the pair costs no
  // HBM bytes there); from kMlpHiOnlyRows rows on, where the products are
  // matrix-core bound, they enter as plain bf16.  The queries and the O
  // product's input keep the pair at every size; the Q/K/V input (measured
  // worth nothing in the hidden error at batch 1, 32 and the 32k context)
  // is plain bf16 with bf16 storage, a pair with fp32 storage.
  const bool mlp_lo = M < kMlpHiOnlyRows;
  const bool qkv_lo = c->storage() == ST_F32;
  // The embedding and the row-tile finishes store the normalised residual for
  // the next Q/K/V, gate/up or LM-head product in fragment blocks when that
  // product runs on the LDS-DMA kernel (each stage's activation loads then
  // move whole 128-byte lines).
  const bool blk = act_blocked(c->storage(), M);
  // the main kernel of a layer product, timed on its own under DFLASH_STAGE_LAYER_GEMM
  auto layer_gemm = [&](GemmArgs& a, bool lo, int N, int K, GemmLaunch* gl) {
    StageScope sc(c, DFLASH_STAGE_LAYER_GEMM, s);
    return gemm_partial(c, a, SRC_SPLIT, lo, M, N, K, gl, s);
  };
  for (int l = 0; l < cf.n_layers; ++l) {
    {  // RMSNorm -> Q/K/V, RoPE
      StageScope sc(c, DFLASH_STAGE_QKV, s);
      GemmArgs a{};
      GemmLaunch gl{};
      a.wt = c->at<void>(L.wt_qkv[l]);
      a.a_hi = xs_hi;
      a.a_lo = qkv_lo ? xs_lo : nullptr;
      a.lda = H;
      a.a_blocked = blk;
      FinishArgs f{};
      norm(a, f);
      if ((st = layer_gemm(a, qkv_lo, Nq + 2 * Nk, H, &gl))) return st;
      f.rope = c->at<float2>(L.rope);
      f.max_ctx = cf.max_ctx;
      f.block = cf.block;
      f.ctx_len = c->ctx_len;
      f.head_dim = D;
      f.n_q_heads = cf.n_q_heads;
      f.n_kv_heads = cf.n_kv_heads;
      f.q_scale = (float)(1.4426950408889634 / std::sqrt((double)D));
      f.out_hi = c->at<void>(L.q_hi);
      f.out_lo = c->at<void>(L.q_lo);
      f.kv_cache[0] = c->kv_k[l];
      f.kv_cache[1] = c->kv_v[l];
      f.kv_int8 = cf.kv_dtype == DFLASH_KV_INT8;
      f.kv_scale[0] = c->kv_ks[l];
      f.kv_scale[1] = c->kv_vs[l];
      f.err = c->at<uint32_t>(L.err);
      if ((st = finish(c, FIN_QKV, f, gl, M, Nq + 2 * Nk, s))) return st;
    }
    {  // attention over [context ; block]
      StageScope sc(c, DFLASH_STAGE_ATTN, s);
      AttnArgs a{};
      a.q_hi = c->at<void>(L.q_hi);
      a.q_lo = c->at<void>(L.q_lo);
      a.kc = c->kv_k[l];
      a.vc = c->kv_v[l];
      a.kv_int8 = cf.kv_dtype == DFLASH_KV_INT8;
      a.ks = c->kv_ks[l];
      a.vs = c->kv_vs[l];
      a.ctx_len = c->ctx_len;
      a.Bs = cf.block;
      a.Hq = cf.n_q_heads;
      a.Hkv = cf.n_kv_heads;
      a.D = D;
      a.max_ctx = cf.max_ctx;
      attn_grid(cf, batch, &a);
      a.p_lo = mlp_lo;
      a.part_o = c->at<float>(L.part_o);
      a.part_ml = c->at<float>(L.part_ml);
      a.seg_info = c->at<int2>(L.seg);
      a.out_hi = c->at<void>(L.o_hi);
      a.out_lo = c->at<void>(L.o_lo);
      a.batch = batch;
      if ((st = hip_status(launch_attention(c->storage(), a, s), "attention launch"))) return st;
    }
    {  // O projection + residual (+ block conv); hi/lo of x * g_post, sums of squares
      StageScope sc(c, DFLASH_STAGE_OPROJ, s);
      GemmArgs a{};
      GemmLaunch gl{};
      a.wt = c->at<void>(L.wt_o[l]);
      a.a_hi = c->at<void>(L.o_hi);
      a.a_lo = c->at<void>(L.o_lo);
      a.lda = Nq;
      if ((st = layer_gemm(a, true, H, Nq, &gl))) return st;
      FinishArgs f{};
      f.x = x;
      f.conv = c->conv[l];
      f.block = cf.block;
      f.gnext = c->g_post[l];
      f.out_hi = xs_hi;
      f.out_lo = mlp_lo ? xs_lo : nullptr;
      f.out_blocked = blk;
      f.ssq_out = ssq;
      f.ld_ssq = L.mmax;
      if ((st = finish(c, FIN_ROWTILE, f, gl, M, H, s))) return st;
    }
    ssq_parts = H / 16;
    {  // RMSNorm -> gate/up, SiLU product
      StageScope sc(c, DFLASH_STAGE_GATEUP, s);
      GemmArgs a{};
      GemmLaunch gl{};
      a.wt = c->at<void>(L.wt_gu[l]);
      a.a_hi = xs_hi;
      a.a_lo = mlp_lo ? xs_lo : nullptr;
      a.lda = H;
      a.a_blocked = blk;
      FinishArgs f{};
      norm(a, f);
      if (!mlp_lo && plan_swiglu(c->storage(), M, F, H, &a, &gl)) {
        // the SiLU product in the main kernel's epilogue (row scales from the sums of squares there)
        StageScope sc2(c, DFLASH_STAGE_LAYER_GEMM, s);
        a.rinv_out = nullptr;
        a.act_out = c->at<void>(L.act_hi);
        a.ld_act = F;
        a.up_tile0 = F / 16;
        if ((st = hip_status(launch_gemm(c->storage(), a, gl, s), "gate/up launch"))) return st;
      } else {
        if ((st = layer_gemm(a, mlp_lo, 2 * F, H, &gl))) return st;
        f.out_hi = c->at<void>(L.act_hi);
        f.out_lo = mlp_lo ? c->at<void>(L.act_lo) : nullptr;
        if ((st = finish(c, FIN_SWIGLU, f, gl, M, 2 * F, s))) return st;
      }
    }
    {  // down projection + residual; hi/lo of x * (next layer's g_in, or g_final)
      StageScope sc(c, DFLASH_STAGE_DOWN, s);
      GemmArgs a{};
      GemmLaunch gl{};
      a.wt = c->at<void>(L.wt_down[l]);
      a.a_hi = c->at<void>(L.act_hi);
      a.a_lo = mlp_lo ? c->at<void>(L.act_lo) : nullptr;
      a.lda = F;
      if ((st = layer_gemm(a, mlp_lo, H, F, &gl))) return st;
      FinishArgs f{};
      f.x = x;
      f.block = cf.block;
      f.gnext = l + 1 < cf.n_layers ? c->g_in[l + 1] : c->g_final;
      f.out_hi = xs_hi;
      f.out_lo = qkv_lo ? xs_lo : nullptr;
      f.out_blocked = blk;
      f.ssq_out = ssq;
      f.ld_ssq = L.mmax;
      if ((st = finish(c, FIN_ROWTILE, f, gl, M, H, s))) return st;
    }
  }
  if (hidden_dbg) {
    if ((st = hip_status(launch_copy_f32(x, hidden_dbg, (size_t)M * H, s), "hidden copy"))) return st;
  }
  GemmLaunch lm{};
  {  // final RMSNorm -> LM head -> per-tile argmax (the positive row scale does not move the argmax)
    StageScope sc(c, DFLASH_STAGE_LMHEAD, s);
    GemmArgs a{};
    GemmLaunch gl{};
    a.wt = c->at<void>(L.wt_lm);
    a.a_hi = xs_hi;
    a.lda = H;
    a.a_blocked = blk;
    a.best_part = c->at<uint64_t>(L.lm_best);
    a.ld_best = M;
    a.logits_dbg = logits_dbg;
    a.ssq_in = ssq;
    a.ssq_nparts = ssq_parts;
    a.ld_ssq = L.mmax;
    a.eps = cf.rms_eps;
    // hi only: the logits feed an argmax and the logit bar, not the residual stream
    if (!plan_gemm(c->storage(), SRC_SPLIT, OUT_ARGMAX, false, M, cf.vocab, H, &a, &gl))
      return fail(DFLASH_EUNSUPPORTED, "no LM-head launch plan");
    if ((st = hip_status(launch_gemm(c->storage(), a, gl, s), "LM head launch"))) return st;
    lm = gl;
  }
  // argmax over the tiles' keys -> draft ids
  return hip_status(launch_argmax_reduce(c->at<uint64_t>(L.lm_best), lm.argmax_tiles, M, M, draft_ids, s),
                    "argmax reduce launch");
}

dflash_status dflash_check(dflash_ctx* c, uint32_t* error_bits, void* stream) {
  g_last_error.clear();
  if (!c || !error_bits) return fail(DFLASH_EINVAL, "null argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, c->at<uint32_t>(c->L.err), 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "error word read");
  *error_bits = v;
  if (v) return fail(DFLASH_EDEVICE, "device error word is set");
  return DFLASH_OK;
}

dflash_status dflash_clear_errors(dflash_ctx* c, void* stream) {
  g_last_error.clear();
  if (!c) return fail(DFLASH_EINVAL, "null context");
  return hip_status(launch_clear_u32(c->at<uint32_t>(c->L.err), 1, static_cast<hipStream_t>(stream)), "clear");
}

dflash_status dflash_stats(dflash_ctx* c, uint64_t out3[3], void* stream) {
  g_last_error.clear();
  if (!c || !out3) return fail(DFLASH_EINVAL, "null argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(out3, c->at<uint64_t>(c->L.stats), 24, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return hip_status(e, "stats read");
}

dflash_status dflash_stage_timing(dflash_ctx* c, int32_t stage, int32_t enable) {
  g_last_error.clear();
  if (!c) return fail(DFLASH_EINVAL, "null context");
  if (stage < 0 || stage >= DFLASH_N_STAGES) return fail(DFLASH_EINVAL, "bad stage");
  EventPool& p = c->timing[stage];
  if (enable && p.begin.empty()) {
    const size_t n = 4096;
    p.begin.resize(n);
    p.end.resize(n);
    for (size_t i = 0; i < n; ++i) {
      hipError_t e = hipEventCreate(&p.begin[i]);
      if (e == hipSuccess) e = hipEventCreate(&p.end[i]);
      if (e != hipSuccess) return hip_status(e, "event create");
    }
  }
  p.enabled = enable != 0;
  return DFLASH_OK;
}

dflash_status dflash_stage_time(dflash_ctx* c, int32_t stage, double* mean_ms, int64_t* count, void* stream) {
  g_last_error.clear();
  if (!c || !mean_ms || !count) return fail(DFLASH_EINVAL, "null argument");
  if (stage < 0 || stage >= DFLASH_N_STAGES) return fail(DFLASH_EINVAL, "bad stage");
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "sync");
  EventPool& p = c->timing[stage];
  double total = 0.0;
  for (size_t i = 0; i < p.used; ++i) {
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, p.begin[i], p.end[i]);
    if (e != hipSuccess) return hip_status(e, "event time");
    total += ms;
  }
  *count = (int64_t)p.used;
  *mean_ms = p.used ? total / (double)p.used : 0.0;
  p.used = 0;
  return DFLASH_OK;
}

void dflash_destroy(dflash_ctx* c) {
  if (!c) return;
  for (auto& p : c->timing) {
    for (auto ev : p.begin) (void)hipEventDestroy(ev);
    for (auto ev : p.end) (void)hipEventDestroy(ev);
  }
  delete c;
}

}  // extern "C"
