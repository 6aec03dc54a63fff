// Launch interface between the C-ABI layer (api.cpp) and the gfx950 kernels.
// Plain structs only; every launcher enqueues on `stream` and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

enum StorageType { ST_F32 = 0, ST_BF16 = 1 };

// ------------------------------------------------------------------ GEMM
// Y[M, N] = A[M, K] . W[N, K]^T with a fused prologue (how the bf16 A operand
// is formed) and epilogue (what is done with the fp32 result tile).
enum ProKind {
  PRO_SPLIT = 0,   // A = a_hi + a_lo, two bf16 arrays [M, lda]; with ssq_in set, result
                   //   rows are scaled by rinv[m] = 1/sqrt(sum_p ssq[p][m] / K + eps)
  PRO_CONCAT = 1   // A: concat of n_src arrays [M, src_width] of storage type S
};
enum EpiKind {
  EPI_F32_SSQ = 0,  // out fp32 [M, ldo] = Y; ssq_out[tile][m] = sum over the tile's columns of Y^2
  EPI_KV = 1,       // context K/V: RoPE on K segments, scatter to the per-layer caches
  EPI_QKV = 2,      // block Q/K/V: RoPE on Q and K, Q scaled, store Q (bf16), K/V (S)
  EPI_RESID = 3,    // x[m, n] += Y (+ width-3 block conv); ssq_out of the new x
  EPI_SWIGLU = 4,   // act[m, f] = bf16(silu(Y_gate) * Y_up)
  EPI_ARGMAX = 5    // per row: running (max, index) over the vocabulary -> draft ids
};

constexpr int kMaxSeg = 16;

struct GemmArgs {
  int M, N, K;
  int WN, WK;  // waves per workgroup along N (16 rows each) and along K
  int P;       // pair stride in rows (0: each tile is NT contiguous rows)
  int kw;      // K per wave
  // W row segments: global row n in [seg_start[s], seg_start[s+1]) is row
  // n - seg_start[s] of matrix seg_ptr[s] (all with row length K).
  int nseg;
  const void* seg_ptr[kMaxSeg];
  int seg_start[kMaxSeg + 1];

  // prologue
  const void* a_hi;  // PRO_SPLIT bf16 [M, lda]
  const void* a_lo;
  int lda;
  const void* src[8];  // PRO_CONCAT sources, each [M, src_width]
  int n_src, src_width;
  const float* ssq_in;  // PRO_SPLIT row scale: partial sums of squares [nparts][ld_ssq] or null
  int ssq_nparts, ld_ssq;
  float eps;

  // epilogue
  float* out_f32;   // EPI_F32_SSQ output [M, N]
  void* out_hi;     // bf16 hi/lo outputs: EPI_F32_SSQ / EPI_RESID (value * gnext), [M, N];
  void* out_lo;     //   EPI_SWIGLU [M, N/2]; EPI_QKV query [M, Hq*D] (RoPE, scaled)
  const void* gnext;  // EPI_F32_SSQ / EPI_RESID: gain of the consumer's RMSNorm [N] (storage type)
  float* ssq_out;   // EPI_F32_SSQ / EPI_RESID: [ntiles][ld_ssq]
  float* x;         // EPI_RESID residual stream fp32 [M, N]
  const void* conv;  // EPI_RESID: [N, 3] taps (storage type) or null
  int block;         // rows per sequence (Bs for the draft, t_new for fuse)
  const int32_t* ctx_len;
  int max_ctx;
  float rope_theta;
  int head_dim;
  int n_q_heads, n_kv_heads;
  float q_scale;
  void* kb_out;  // EPI_QKV storage type [M, Hkv*D]
  void* vb_out;
  void* kv_cache[kMaxSeg];  // EPI_KV: one cache per segment (K^0, V^0, K^1, V^1, ...)
  uint32_t* err;
  uint64_t* best_part;  // EPI_ARGMAX per-tile packed (value, index) keys [ntiles][ld_best]
  int ld_best;
  float* logits_dbg;    // EPI_ARGMAX nullable [M, N]
};

struct GemmLaunch {
  int MR;       // 16-row m-subtiles per workgroup
  int mtiles;   // grid.y
  int ntiles;   // grid.x
  int threads;  // 64 * WN * WK
  size_t lds;   // dynamic LDS bytes
};

hipError_t launch_gemm(int storage, ProKind pro, EpiKind epi, const GemmArgs& a, const GemmLaunch& l,
                       hipStream_t stream);
size_t gemm_lds_bytes(EpiKind epi, int MR, int WN, int WK);
// ids[m] = index of the largest key over part[t][m], t < ntiles.
hipError_t launch_argmax_reduce(const uint64_t* part, int ntiles, int ld, int M, int32_t* ids, hipStream_t stream);
int gemm_max_threads(int storage, ProKind pro, int MR);

// ------------------------------------------------------------------ attention
struct AttnArgs {
  const void* q_hi;  // bf16 hi/lo pair [B*Bs, Hq*D], already scaled by log2(e)/sqrt(D)
  const void* q_lo;
  const void* kb;  // storage [B*Bs, Hkv*D] block keys (RoPE applied)
  const void* vb;
  const void* kc;  // storage [B, max_ctx, Hkv, D] this layer's cache
  const void* vc;
  const int32_t* ctx_len;
  int Bs, Hq, Hkv, D, max_ctx;
  int CW;          // keys per split
  int max_splits;  // grid.x
  float* part_o;   // [B*Hkv*max_splits, QR, D]   unnormalised split outputs
  float* part_ml;  // [B*Hkv*max_splits, QR, 2]   split running max and sum
  void* out_hi;    // bf16 hi/lo pair [B*Bs, Hq*D]
  void* out_lo;
  int batch;
};
// Launches the split attention and, for sequences with more than one split,
// the merge of the split partials.
hipError_t launch_attention(int storage, const AttnArgs& a, hipStream_t stream);

// ------------------------------------------------------------------ small kernels
struct VerifyArgs {
  const float* logits;  // [batch, n_d+1, V]
  const int32_t* draft;
  int draft_stride, n_d, batch, V, max_ctx;
  int chunk;        // vocab entries per workgroup of the streaming pass
  int nchunks;
  uint64_t* part;   // [batch*(n_d+1)][nchunks] packed (value, index) keys
  int32_t* n_accept;
  int32_t* bonus;
  int32_t* out_tokens;
  int32_t* ctx_len;
  unsigned long long* stats;  // {steps, accepted, drafted}
  uint32_t* err;
};
// Two launches: the streaming argmax over the target logits, then the
// per-sequence accepted prefix, bonus token, commit and counters.
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);

hipError_t launch_embed(int storage, const void* embed, const void* gain, const int32_t* ids, int M, int H, int V,
                        float* x, void* xs_hi, void* xs_lo, float* ssq, uint32_t* err, hipStream_t stream);
hipError_t launch_commit(int32_t* ctx_len, int batch, int t_new, int max_ctx, hipStream_t stream);
hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t stream);
hipError_t launch_feature_dbg(int storage, const float* y, const float* ssq, int nparts, int ld_ssq,
                              const void* gain, float eps, int M, int H, float* out, hipStream_t stream);
hipError_t launch_clear_u32(uint32_t* p, int n, hipStream_t stream);

}  // namespace dfl
