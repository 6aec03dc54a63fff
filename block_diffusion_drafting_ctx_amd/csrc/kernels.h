// Launch interface between the C-ABI layer (api.cpp) and the gfx950 kernels.
// Plain structs only; every launcher enqueues on `stream` and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

enum StorageType { ST_F32 = 0, ST_BF16 = 1 };

// Device error-word bits (the public header's DFLASH_ERR_*).
constexpr uint32_t kErrFuseOverflow = 1u << 0;    // ctx_len + t_new > max_ctx in the fusion
constexpr uint32_t kErrTokenRange = 1u << 1;      // block id outside [0, vocab)
constexpr uint32_t kErrVerifyOverflow = 1u << 2;  // ctx_len + n_d + 1 > max_ctx in verify
constexpr uint32_t kErrDraftOverflow = 1u << 3;   // ctx_len + block > max_ctx in the draft

// ------------------------------------------------------------------ GEMM
// Y[M, N] = A[M, K] . W[N, K]^T.  The N axis concatenates weight matrices
// (one tiled bf16 buffer per product) and is cut into 16-row tiles.  The main kernel writes fp32 partial tiles
// part[k-slice][tile][m][16] (OUT_PARTIAL) that a finish kernel sums and
// post-processes, or per-tile argmax keys (OUT_ARGMAX, one k-slice).
enum SrcKind {
  SRC_SPLIT = 0,   // A = a_hi (+ a_lo): bf16 arrays [M, lda]
  SRC_CONCAT = 1   // A: concat of n_src arrays [M, src_width] of the storage type
};
// OUT_SWIGLU (GEMM_DMA, SRC_SPLIT, one k-slice): N = 2F concatenates gate and
// up; workgroup nb takes gate tiles 6nb.. and the matching up tiles
// up_tile0 + 6nb.., and writes act_out[m, c] = silu(r y_gate) * (r y_up) in
// bf16, r the row's RMSNorm scale summed from ssq_in in the kernel.
enum OutKind { OUT_PARTIAL = 0, OUT_ARGMAX = 1, OUT_SWIGLU = 2 };
enum GemmKind { GEMM_AS = 0, GEMM_MT = 1, GEMM_DMA = 2 };

constexpr int kMaxSeg = 16;  // context K/V caches one product writes (2 per layer)
constexpr size_t kGemmAsSliceLds = 100 * 1024;  // split-K activation slice of a gemm_as workgroup
constexpr size_t kGemmAsMaxLds = 150 * 1024;    // whole-K activation (LM head; one workgroup per CU)

struct GemmArgs {
  int M, N, K;
  // W [N, K] of the product in tiled bf16 (launch_tile_weights): the block of
  // rows 16t.. and columns 32s.. is 1 KB at ((t * K/32 + s) * 64) * 8 elements.
  const void* wt;
  // activations
  const void* a_hi;
  const void* a_lo;
  int lda;
  // SRC_SPLIT on GEMM_DMA only: a_hi / a_lo are stored in fragment blocks
  // (frag_block_index, row length K, rows rounded up to 16; lda unused)
  int a_blocked;
  const void* src[8];
  int n_src, src_width;
  // launch geometry (filled by the planner)
  int ksl, tpw;             // GEMM_AS: k-slice length, tiles per workgroup
  int nbm, nbn, KS, kslice;  // GEMM_MT: M blocks, N blocks, k-slices, k-slice length
  // outputs
  float* part;          // OUT_PARTIAL
  uint64_t* best_part;  // OUT_ARGMAX [argmax tiles][ld_best]
  int ld_best;
  float* logits_dbg;    // OUT_ARGMAX nullable [M, N], row-scaled by rinv
  // RMSNorm of the activation rows: ssq_in[p][m] (p < ssq_nparts, leading
  // dimension ld_ssq) are partial sums of squares over the K columns.
  const float* ssq_in;
  int ssq_nparts, ld_ssq;
  float eps;
  // nullable: workgroup (0, 0) writes rinv_out[m] = 1/sqrt(sum_p ssq_in[p][m]/K + eps)
  // after its tiles, for the finish kernel of this product
  float* rinv_out;
  // OUT_SWIGLU: bf16 [M, ld_act] output, first up tile (F / 16)
  void* act_out;
  int ld_act, up_tile0;
};

struct GemmLaunch {
  int kind;   // GemmKind
  int src, out, lo;
  int MR;
  int NF;  // GEMM_MT: 16-column fragments per wave (block width 32 * NF)
  dim3 grid;
  int threads;
  size_t lds;
  int KS;            // k-slices written (OUT_PARTIAL)
  int argmax_tiles;  // OUT_ARGMAX: key columns per row in best_part (one per workgroup / column block)
};

hipError_t launch_gemm(int storage, const GemmArgs& a, const GemmLaunch& l, hipStream_t stream);
// Weight tiling: rows [0, rows) of the row-major [rows, K] matrix src (storage
// type) become tiles tile0 .. tile0 + rows/16 - 1 of dst, a tiled bf16 matrix
// of row length K: the 16 x 32 block (tile t, k-step s) is stored as the 64
// matrix-core lanes' 16-byte fragments in lane order, lane l holding row
// 16t + (l & 15), columns 32s + 8(l >> 4) .. + 7.  rows % 16 == 0, K % 32 == 0.
hipError_t launch_tile_weights(int storage, const void* src, int rows, int K, void* dst, int tile0,
                               hipStream_t stream);
// k-slice length gemm_as uses for (M, K) over ntiles 16-row tiles on cus
// compute units (0: gemm_as does not fit).
int gemm_as_ksl(int M, int K, bool lo, bool argmax, int ntiles, int cus);
size_t gemm_as_lds(int M, int ksl, bool lo);
// gemm_mt block: BM = 64 * MF rows by BN = 32 * NF columns (NF = 4 for
// MF < 4; 8, or 6 for split-K outputs, at MF = 4); LDS bytes of its stage
// ring (lo: hi/lo activation pair).
size_t gemm_mt_lds_bytes(int MF, int NF, bool lo);
// gemm_dma (64*MF-row blocks, MF = 3 or 4, bf16 operands, stages through
// LDS-DMA): LDS bytes of its stage ring for NF = 6 or 8 (swiglu: with the
// ring of per-stage sums of squares of OUT_SWIGLU).
size_t gemm_dma_lds_bytes(int MF, int NF, bool lo, bool swiglu);
// ids[m] = index of the largest key over part[t][m], t < ntiles.
hipError_t launch_argmax_reduce(const uint64_t* part, int ntiles, int ld, int M, int32_t* ids, hipStream_t stream);

// ------------------------------------------------------------------ GEMM finish
enum FinishKind {
  FIN_ROWTILE = 0,  // y = sum (+ x residual, + block conv): x / out_f32, hi/lo of y*gnext, ssq per tile
  FIN_SWIGLU = 1,   // act = silu(r*gate) * (r*up) as hi/lo
  FIN_QKV = 2,      // RoPE(q, k), q scaled as hi/lo, k and v in storage type
  FIN_KV = 3        // context K/V with RoPE on K into the per-layer caches
};

struct FinishArgs {
  const float* part;
  int KS, ntiles, M, N;
  const float* rinv;  // row scale [M] (written by the product's main kernel); null: none
  int ld_ssq;
  // FIN_ROWTILE
  float* x;           // residual stream [M, N] (read and written) or null
  float* out_f32;     // plain output [M, N] or null
  const void* conv;   // [N, 3] taps (storage type) or null
  const void* gnext;  // [N] gain of the consumer's RMSNorm (storage type)
  float* ssq_out;     // [N/16][ld_ssq]
  void* out_hi;       // FIN_ROWTILE [M, N]; FIN_SWIGLU [M, N/2]; FIN_QKV query [M, Hq*D]
  void* out_lo;       //   (null: hi only)
  int out_blocked;    // FIN_ROWTILE: out_hi / out_lo in fragment blocks (frag_block_index, row length N)
  int block;          // rows per sequence
  // FIN_QKV / FIN_KV
  const float2* rope;  // [max_ctx + max rows per sequence][head_dim / 2] (cos, sin)
  const int32_t* ctx_len;
  int max_ctx;
  int head_dim, n_q_heads, n_kv_heads;
  float q_scale;
  void* kv_cache[kMaxSeg];  // FIN_KV: one per segment; FIN_QKV: this layer's K, V caches
  // 8-bit caches: the values above are int8 and kv_scale[i] holds the float
  // scale of every run of 32 values (flat value index / 32)
  int kv_int8;
  float* kv_scale[kMaxSeg];
  uint32_t* err;
};
hipError_t launch_finish(int storage, FinishKind kind, const FinishArgs& f, hipStream_t stream);

// ------------------------------------------------------------------ attention
// Sequences per attention launch (the per-workgroup prefix table of segment
// lengths lives in LDS).
constexpr int kAttnMaxBatch = 1024;
// Keys of streaming a flattened-split attention workgroup's plan charges for
// every segment it starts (positions on the weighted key axis).
constexpr int kCUs = 256;  // compute units of the chip
constexpr int kAttnPieceCost = 256;
struct AttnArgs {
  const void* q_hi;  // bf16 hi/lo pair [B*Bs, Hq*D], already scaled by log2(e)/sqrt(D)
  const void* q_lo;
  const void* kc;  // storage [B, max_ctx, Hkv, D] this layer's cache; the block's
  const void* vc;  //   K/V (RoPE applied) at rows ctx_len[b] + i
  int kv_int8;        // 8-bit cache: kc/vc are int8 and ks/vs the scales of
  const float* ks;    //   every run of 32 values (flat value index / 32)
  const float* vs;
  const int32_t* ctx_len;
  int Bs, Hq, Hkv, D, max_ctx;
  int nwg;           // workgroups the batch's key axis is cut over (grid of the split kernel)
  int fixed_chunk;   // > 0: fixed chunks of this many keys, fixed_pieces per segment
  int fixed_pieces;  //   (nwg = B * Hkv * fixed_pieces); 0: planned from the lengths
  int p_lo;          // probabilities as a hi/lo pair in the PV product (else plain bf16)
  float* part_o;   // [nwg + B*Hkv slots, QR, D]   unnormalised piece outputs
  float* part_ml;  // [nwg + B*Hkv slots, QR, 2]   piece running max and sum
  int2* seg_info;  // [B*Hkv] planned launches: (first workgroup, pieces) of each segment, for the merge
  void* out_hi;    // bf16 hi/lo pair [B*Bs, Hq*D]
  void* out_lo;
  int batch;
};
// Launches the split attention and the merge of the pieces of every segment
// that more than one workgroup touched.
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
  // sampling mode
  float inv_temp;         // 1 / T
  const float* uniforms;  // [batch, n_d+1, 2]: (accept test, inverse-CDF draw) per row
};
// Two launches: the streaming argmax over the target logits, then the
// per-sequence accepted prefix, bonus token, commit and counters (a null
// stats or err pointer skips the counters / the error bit).
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);
// Keys of the library-owned static scratch the context-free verify uses
// (512 KB per device, for the life of the process).
constexpr size_t kStaticVerifyKeys = 65536;
// Device address of the current device's copy of that scratch (looked up
// once per device with hipGetSymbolAddress, then cached).
hipError_t static_verify_scratch(uint64_t** ptr);
// Sampling mode, two launches: per (row, vocab chunk) the maximum and
// exp-sum of logits / T (kept in the key slots), then per sequence the
// accept tests, the inverse-CDF draw of the emitted token, commit, counters.
// a.chunk must be 4 * 256 * 8 (one 16-byte load round per thread).
hipError_t launch_verify_sample(const VerifyArgs& a, hipStream_t stream);

// blocked: xs_hi / xs_lo in fragment blocks (frag_block_index), else
// row-major; xs_lo may be null (hi only).  ssq receives H/128 partial sums of
// squares per row ([slice][ld_ssq]).  H % 128 == 0.
hipError_t launch_embed(int storage, const void* embed, const void* gain, const int32_t* ids, int M, int H, int V,
                        float* x, void* xs_hi, void* xs_lo, bool blocked, float* ssq, int ld_ssq, uint32_t* err,
                        hipStream_t stream);
hipError_t launch_commit(int32_t* ctx_len, int batch, int t_new, int max_ctx, hipStream_t stream);
// table[p][i] = (cos, sin)(p * theta^(-2i/D)), evaluated in double precision.
hipError_t launch_rope_table(float2* table, int rows, int head_dim, float theta, hipStream_t stream);
hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t stream);
hipError_t launch_feature_dbg(int storage, const float* y, const float* ssq, int nparts, int ld_ssq,
                              const void* gain, float eps, int M, int H, float* out, hipStream_t stream);
hipError_t launch_clear_u32(uint32_t* p, int n, hipStream_t stream);

// Raises the dynamic-LDS limit of `kernel` on the current device to `bytes`
// (needed above 64 KB).  The runtime call is made once per (device, kernel)
// and larger size; later calls are a table lookup.
hipError_t allow_dynamic_lds(const void* kernel, size_t bytes);

}  // namespace dfl
