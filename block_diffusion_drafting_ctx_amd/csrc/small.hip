// Verify (greedy target argmax + accepted prefix + commit), block embedding,
// context commit and small helpers.  Cross-workgroup results always go
// through plain stores and a following kernel: a fence-and-ticket handoff
// costs tens of nanoseconds per workgroup on this chip.
#include <map>
#include <mutex>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace dfl {

// ---------------------------------------------------------------- verify
// Pass 1, grid (vocab chunks, rows = batch*(n_d+1)), 256 threads: stream the
// target logits once (16-byte non-temporal loads, 8 per thread issued
// together) and fold (value, index) into one packed key per (row, chunk) --
// order independent, so the result is exact.
__global__ void __launch_bounds__(256) verify_argmax_kernel(const VerifyArgs a) {
  __shared__ uint64_t s_best[4];
  constexpr int PER = 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.y;
  const int v0 = blockIdx.x * a.chunk;
  const int v1 = min(a.V, v0 + a.chunk);
  const float* p = a.logits + (size_t)row * a.V;
  uint64_t best = 0;
  for (int vb = v0; vb < v1; vb += 4 * 256 * PER) {
    f32x4 x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = vb + 4 * (tid + 256 * i);  // V is a multiple of 64: a piece never straddles v1
      if (v < v1) x[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + v));
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = vb + 4 * (tid + 256 * i);
      if (v >= v1) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t k = argmax_key(x[i][e], (uint32_t)(v + e));
        best = k > best ? k : best;
      }
    }
  }
  best = wave_max_u64(best);
  if (lane == 0) s_best[wave] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t bb = s_best[0];
    for (int w = 1; w < 4; ++w) bb = s_best[w] > bb ? s_best[w] : bb;
    a.part[(size_t)row * a.nchunks + blockIdx.x] = bb;
  }
}

// Pass 2, one workgroup per sequence: greedy tokens g_i, accepted prefix n,
// bonus g_n, committed tokens, context-length advance (rollback of the rest)
// and the step counters.
__global__ void __launch_bounds__(64) verify_commit_kernel(const VerifyArgs a) {
  __shared__ int s_g[65], s_d[64];
  __shared__ int s_n;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int R = a.n_d + 1;
  const int32_t* d = a.draft + (size_t)b * a.draft_stride;
  for (int i = tid; i < R; i += 64) {
    // the draft ids are loaded alongside the keys, so the comparison below
    // runs from LDS instead of one dependent global load per accepted token
    if (i < a.n_d) s_d[i] = d[i];
    const uint64_t* pr = a.part + ((size_t)b * R + i) * a.nchunks;
    uint64_t best = 0;
    for (int c = 0; c < a.nchunks; ++c) best = pr[c] > best ? pr[c] : best;
    s_g[i] = argmax_key_index(best);
  }
  __syncthreads();
  if (tid == 0) {
    int n = 0;
    while (n < a.n_d && s_d[n] == s_g[n]) ++n;
    s_n = n;
    a.n_accept[b] = n;
    a.bonus[b] = s_g[n];
    const int t0 = a.ctx_len[b];
    if (t0 < 0 || t0 + R > a.max_ctx) {
      if (a.err) atomicOr(a.err, kErrVerifyOverflow);
    } else {
      a.ctx_len[b] = t0 + n + 1;
    }
    if (a.stats) {
      atomicAdd(&a.stats[0], 1ull);
      atomicAdd(&a.stats[1], (unsigned long long)n);
      atomicAdd(&a.stats[2], (unsigned long long)a.n_d);
    }
  }
  __syncthreads();
  for (int i = tid; i < R; i += 64) a.out_tokens[(size_t)b * R + i] = i <= s_n ? s_g[i] : -1;
}

// ---------------------------------------------------------------- library-owned scratch
// For callers that cannot allocate device memory: the (row, vocabulary chunk)
// argmax keys of the context-free greedy verify live in this array, one copy
// per device for the life of the process.  Every call on a device shares it
// (and keeps the last call's keys; each key is written before it is read, so
// nothing needs clearing): calls that overlap on one device race.
static __device__ __align__(256) uint64_t scratch[kStaticVerifyKeys];

hipError_t static_verify_scratch(uint64_t** ptr) {
  static std::mutex mu;
  static std::map<int, uint64_t*> addr;  // device -> device address of its copy of `scratch`
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    it = addr.emplace(dev, static_cast<uint64_t*>(p)).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
  dim3 grid(a.nchunks, a.batch * (a.n_d + 1)), block(256);
  hipLaunchKernelGGL(verify_argmax_kernel, grid, block, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_commit_kernel, dim3(a.batch), dim3(64), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- verify, sampling mode
// Pass 1, grid (vocab chunks, rows), 256 threads: the chunk's logits z = x / T
// (one round of 8 16-byte loads a thread covers the 8192-entry chunk), its
// maximum m and s = sum exp(z - m), both reduced in a fixed order, stored as
// a float pair in the (row, chunk) key slot.  A NaN logit carries no mass
// (it is read as -inf).
__global__ void __launch_bounds__(256) verify_stats_kernel(const VerifyArgs a) {
  __shared__ float s_red[4];
  constexpr int PER = 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.y;
  const int v0 = blockIdx.x * a.chunk;
  const int v1 = min(a.V, v0 + a.chunk);
  const float* p = a.logits + (size_t)row * a.V;
  float z[PER][4];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int v = v0 + 4 * (tid + 256 * i);  // V is a multiple of 64: a piece never straddles v1
    f32x4 x = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (v < v1) x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + v));
#pragma unroll
    for (int e = 0; e < 4; ++e) z[i][e] = v < v1 && x[e] == x[e] ? x[e] * a.inv_temp : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, z[i][e]);
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) sum += z[i][e] == -INFINITY ? 0.f : __expf(z[i][e] - m);
  sum = wave_sum_f32(sum);
  if (lane == 0) s_red[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    const float2 ms = make_float2(m, ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3]);
    a.part[(size_t)row * a.nchunks + blockIdx.x] = __builtin_bit_cast(uint64_t, ms);
  }
}

// Pass 2, one 256-thread workgroup per sequence.  Rows i < n_d accept draft
// d_i while u[i][0] < p_i(d_i), p_i = softmax(x_i / T); the token emitted at
// row n (the first rejection, with d_n removed from the distribution, or the
// bonus row n_d) is the inverse CDF of p_n at u[n][1], over the vocabulary in
// index order: whole chunks first from the pass-1 sums, then a prefix scan
// inside the chunk that holds it.  Every step is wave-parallel: the reads that
// do not depend on one another are issued together, each row's sums are a
// wave reduction, the accepted prefix is a ballot and both prefix sums are
// wave scans.
constexpr int kSamplePartLds = 2560;  // (row, chunk) partials staged in LDS, e.g. 65 rows x 39 chunks

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
// inclusive prefix sum over the lanes of a wave, in lane order
__device__ __forceinline__ float wave_scan_f32(float v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  return v;
}
// mass of a (max, exp-sum) partial relative to the row maximum M; an empty
// or all -inf chunk carries none
__device__ __forceinline__ float part_mass(float2 ms, float M) { return ms.y > 0.f ? ms.y * __expf(ms.x - M) : 0.f; }

__global__ void __launch_bounds__(256) verify_sample_commit_kernel(const VerifyArgs a) {
  __shared__ float2 s_part[kSamplePartLds];
  __shared__ float s_M[65], s_S[65], s_xd[64], s_pd[64], s_u[130], s_wsum[4];
  __shared__ int s_d[64], s_n, s_ex, s_chunk, s_tok;
  __shared__ float s_t;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = a.n_d + 1, NC = a.nchunks;
  const int32_t* d = a.draft + (size_t)b * a.draft_stride;
  const float2* gpart = reinterpret_cast<const float2*>(a.part) + (size_t)b * R * NC;
  const bool staged = R * NC <= kSamplePartLds;
  // independent reads, all in flight at once: the partials, the uniforms,
  // the draft ids and the logit of each draft (-inf outside the vocabulary
  // or at a NaN logit: such a draft is never accepted)
  if (staged)
    for (int k = tid; k < R * NC; k += 256) s_part[k] = gpart[k];
  if (tid < 2 * R) s_u[tid] = a.uniforms[(size_t)b * R * 2 + tid];
  if (tid < a.n_d) {
    const int di = d[tid];
    s_d[tid] = di;
    const float xd = di >= 0 && di < a.V ? a.logits[((size_t)b * R + tid) * a.V + di] : -INFINITY;
    s_xd[tid] = xd == xd ? xd * a.inv_temp : -INFINITY;
  }
  __syncthreads();
  const float2* part = staged ? s_part : gpart;
  for (int i = wave; i < R; i += 4) {  // row i: maximum M and sum S of exp(x / T - M)
    const float2* pr = part + i * NC;
    float M = -INFINITY;
    for (int c = lane; c < NC; c += 64) M = fmaxf(M, pr[c].x);
    M = wave_max_f32(M);
    float S = 0.f;
    for (int c = lane; c < NC; c += 64) S += part_mass(pr[c], M);
    S = wave_sum_f32(S);
    if (lane == 0) {
      s_M[i] = M;
      s_S[i] = S;
      if (i < a.n_d) s_pd[i] = __expf(s_xd[i] - M) / S;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const bool acc = lane < a.n_d && s_u[2 * lane] < s_pd[lane];
    const uint64_t rej = ~__ballot(acc);
    const int n = min(a.n_d, rej ? (int)__builtin_ctzll(rej) : 64);
    const int ex = n < a.n_d && s_d[n] >= 0 && s_d[n] < a.V ? s_d[n] : -1;  // the rejected draft leaves the draw
    const float M = s_M[n];
    const float wex = ex >= 0 ? __expf(s_xd[n] - M) : 0.f;
    const float t = s_u[2 * n + 1] * (s_S[n] - wex);
    const float2* pr = part + n * NC;
    // the first chunk whose inclusive prefix of mass exceeds t
    int chunk = -1, last = 0;
    float rest = INFINITY, carry = 0.f;
    for (int c0 = 0; c0 < NC; c0 += 64) {
      const int c = c0 + lane;
      float w = 0.f;
      if (c < NC) {
        w = part_mass(pr[c], M);
        if (ex >= c * a.chunk && ex < (c + 1) * a.chunk) w -= wex;
      }
      const float incl = carry + wave_scan_f32(w, lane);
      const uint64_t pos = __ballot(c < NC && w > 0.f);
      if (pos) last = c0 + 63 - (int)__builtin_clzll(pos);
      const uint64_t hit = __ballot(c < NC && t < incl);
      if (hit) {
        const int src = (int)__builtin_ctzll(hit);
        chunk = c0 + src;
        rest = t - __shfl(incl - w, src);
        break;
      }
      carry = __shfl(incl, 63);
    }
    if (chunk < 0) chunk = last;  // rounding left t at the top: the last chunk holding mass, rest = inf
    if (lane == 0) {
      s_n = n;
      s_ex = ex;
      s_chunk = chunk;
      s_t = rest;
      s_tok = -1;
    }
  }
  __syncthreads();
  // inside the chunk: thread tid takes 32 consecutive entries (V and the
  // chunk are multiples of 64, so a thread's run is wholly in or out)
  const int j = s_n, ex = s_ex;
  const float* xj = a.logits + ((size_t)b * R + j) * a.V;
  const float Mj = s_M[j];
  const int v0 = s_chunk * a.chunk + 32 * tid;
  const bool in = v0 < min(a.V, (s_chunk + 1) * a.chunk);
  float e[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    f32x4 x = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (in) x = *reinterpret_cast<const f32x4*>(xj + v0 + 4 * q);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      e[4 * q + r] = v0 + 4 * q + r != ex && x[r] == x[r] ? __expf(x[r] * a.inv_temp - Mj) : 0.f;
  }
  float mine = 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) mine += e[k];
  const float incl = wave_scan_f32(mine, lane);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  float lo = incl - mine;
  for (int w = 0; w < wave; ++w) lo += s_wsum[w];
  const float t = s_t;
  if (t >= lo && t < lo + mine) {
    float run = lo;
    int tok = -1;
    for (int k = 0; k < 32 && tok < 0; ++k) {
      run += e[k];
      if (t < run && e[k] > 0.f) tok = v0 + k;
    }
    if (tok >= 0) s_tok = tok;
  }
  __syncthreads();
  if (s_tok < 0) {  // rounding: the last entry of the chunk holding mass
    int best = -1;
#pragma unroll
    for (int k = 0; k < 32; ++k)
      if (e[k] > 0.f) best = v0 + k;
    const unsigned long long key = best < 0 ? 0ull : (unsigned long long)(best + 1);
    __shared__ unsigned long long s_last;
    if (tid == 0) s_last = 0ull;
    __syncthreads();
    atomicMax(&s_last, key);
    __syncthreads();
    if (tid == 0) s_tok = (int)s_last - 1;
    __syncthreads();
  }
  if (tid == 0) {
    const int n = s_n, tok = s_tok;
    a.n_accept[b] = n;
    a.bonus[b] = tok;
    const int t0 = a.ctx_len[b];
    if (t0 < 0 || t0 + R > a.max_ctx) {
      atomicOr(a.err, kErrVerifyOverflow);
    } else {
      a.ctx_len[b] = t0 + n + 1;
    }
    atomicAdd(&a.stats[0], 1ull);
    atomicAdd(&a.stats[1], (unsigned long long)n);
    atomicAdd(&a.stats[2], (unsigned long long)a.n_d);
  }
  for (int i = tid; i < R; i += 256)
    a.out_tokens[(size_t)b * R + i] = i < s_n ? d[i] : (i == s_n ? s_tok : -1);
}

hipError_t launch_verify_sample(const VerifyArgs& a, hipStream_t stream) {
  if (a.chunk != 4 * 256 * 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(verify_stats_kernel, dim3(a.nchunks, a.batch * (a.n_d + 1)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_sample_commit_kernel, dim3(a.batch), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- embedding
// x[m] = E[ids[m]] as fp32, the hi/lo pair of x * gain (the first layer's
// RMSNorm gain; row-major or in fragment blocks; a null xs_lo: hi only) and
// the row's sums of squares, one partial per 128-column slice
// (ssq[slice * ld_ssq + m]).  grid: (16-row groups, H/128 slices); thread t
// takes row t / 16 of the group and columns 8 (t % 16) .. + 7 of the slice,
// so a workgroup writes whole 16 x 32 fragment blocks.
template <typename S>
__global__ void __launch_bounds__(256) embed_kernel(const S* embed, const S* gain, const int32_t* ids, int M, int H,
                                                    int V, float* x, bf16_t* xs_hi, bf16_t* xs_lo, int blocked,
                                                    float* ssq, int ld_ssq, uint32_t* err) {
  const int tid = threadIdx.x, m = 16 * blockIdx.x + (tid >> 4), k = 128 * blockIdx.y + 8 * (tid & 15);
  const bool live = m < M;
  const int id = live ? ids[m] : 0;
  const bool ok = id >= 0 && id < V;
  if (live && !ok && blockIdx.y == 0 && (tid & 15) == 0) atomicOr(err, kErrTokenRange);
  Raw8 raw, graw;
  load_raw8<S>(raw, embed + (size_t)(ok ? id : 0) * H + k);
  load_raw8<S>(graw, gain + k);
  float f[8], gf[8];
  raw_to_f32x8<S>(raw, f);
  raw_to_f32x8<S>(graw, gf);
  uint32_t hw[4], lw[4];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[i] = ok ? f[i] : 0.f;
    s += f[i] * f[i];
    const float v = f[i] * gf[i];
    const uint32_t hbits = f32_to_bf16_bits(v);
    const uint32_t lbits = f32_to_bf16_bits(v - bf16_bits_to_f32(hbits));
    hw[i >> 1] = (i & 1) ? hw[i >> 1] | hbits << 16 : hbits;
    lw[i >> 1] = (i & 1) ? lw[i >> 1] | lbits << 16 : lbits;
  }
  // the row's 16 lanes (a 16-lane group of one wave)
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o);
  if (!live) return;
  // the 8 columns k .. k+7 are one 16-byte piece in either layout
  const size_t idx = blocked ? frag_block_index(m, k, H) : (size_t)m * H + k;
  *reinterpret_cast<u32x4*>(xs_hi + idx) = u32x4{hw[0], hw[1], hw[2], hw[3]};
  if (xs_lo != nullptr) *reinterpret_cast<u32x4*>(xs_lo + idx) = u32x4{lw[0], lw[1], lw[2], lw[3]};
  f32x4* dst = reinterpret_cast<f32x4*>(x + (size_t)m * H + k);
  dst[0] = f32x4{f[0], f[1], f[2], f[3]};
  dst[1] = f32x4{f[4], f[5], f[6], f[7]};
  if ((tid & 15) == 0) ssq[(size_t)blockIdx.y * ld_ssq + m] = s;
}

hipError_t launch_embed(int storage, const void* embed, const void* gain, const int32_t* ids, int M, int H, int V,
                        float* x, void* xs_hi, void* xs_lo, bool blocked, float* ssq, int ld_ssq, uint32_t* err,
                        hipStream_t stream) {
  if (H % 128 || M < 1 || ld_ssq < M) return hipErrorInvalidValue;
  const dim3 grid((M + 15) / 16, H / 128);
  if (storage == ST_BF16)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, grid, dim3(256), 0, stream, (const bf16_t*)embed, (const bf16_t*)gain,
                       ids, M, H, V, x, (bf16_t*)xs_hi, (bf16_t*)xs_lo, (int)blocked, ssq, ld_ssq, err);
  else
    hipLaunchKernelGGL(embed_kernel<float>, grid, dim3(256), 0, stream, (const float*)embed, (const float*)gain, ids,
                       M, H, V, x, (bf16_t*)xs_hi, (bf16_t*)xs_lo, (int)blocked, ssq, ld_ssq, err);
  return hipGetLastError();
}

// ---------------------------------------------------------------- commit
__global__ void commit_kernel(int32_t* ctx_len, int batch, int t_new, int max_ctx) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch && ctx_len[b] + t_new <= max_ctx) ctx_len[b] += t_new;
}

hipError_t launch_commit(int32_t* ctx_len, int batch, int t_new, int max_ctx, hipStream_t stream) {
  hipLaunchKernelGGL(commit_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, ctx_len, batch, t_new, max_ctx);
  return hipGetLastError();
}

// ---------------------------------------------------------------- RoPE table
// (cos, sin) of p * theta^(-2i/D) for every position p < rows and pair i < D/2,
// evaluated in double precision and rounded once to fp32.
__global__ void rope_table_kernel(float2* table, int rows, int head_dim, float theta) {
  const int half = head_dim / 2;
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (size_t)rows * half) return;
  const int p = (int)(e / half), i = (int)(e - (size_t)p * half);
  const double inv_freq = exp(-(2.0 * (double)i / (double)head_dim) * log((double)theta));
  double sn, cs;
  sincos((double)p * inv_freq, &sn, &cs);
  table[e] = make_float2((float)cs, (float)sn);
}

hipError_t launch_rope_table(float2* table, int rows, int head_dim, float theta, hipStream_t stream) {
  const size_t n = (size_t)rows * (head_dim / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, table, rows, head_dim,
                     theta);
  return hipGetLastError();
}

// ---------------------------------------------------------------- helpers
__global__ void copy_f32_kernel(const float* src, float* dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t stream) {
  const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(copy_f32_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream, src, dst, n);
  return hipGetLastError();
}

// c = y * rinv * g with rinv from the partial sums of squares (debug output
// of the fused context feature; the same scale the K/V projection applies).
template <typename S>
__global__ void feature_dbg_kernel(const float* y, const float* ssq, int nparts, int ld_ssq, const S* gain,
                                   float eps, int H, float* out) {
  const int m = blockIdx.x;
  float s = 0.f;
  for (int p = 0; p < nparts; ++p) s += ssq[p * ld_ssq + m];
  const float rinv = 1.0f / sqrtf(s / (float)H + eps);
  for (int k = threadIdx.x; k < H; k += blockDim.x)
    out[(size_t)m * H + k] = y[(size_t)m * H + k] * load_f32<S>(gain + k) * rinv;
}

hipError_t launch_feature_dbg(int storage, const float* y, const float* ssq, int nparts, int ld_ssq,
                              const void* gain, float eps, int M, int H, float* out, hipStream_t stream) {
  if (storage == ST_BF16)
    hipLaunchKernelGGL(feature_dbg_kernel<bf16_t>, dim3(M), dim3(256), 0, stream, y, ssq, nparts, ld_ssq,
                       (const bf16_t*)gain, eps, H, out);
  else
    hipLaunchKernelGGL(feature_dbg_kernel<float>, dim3(M), dim3(256), 0, stream, y, ssq, nparts, ld_ssq,
                       (const float*)gain, eps, H, out);
  return hipGetLastError();
}

__global__ void clear_u32_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_clear_u32(uint32_t* p, int n, hipStream_t stream) {
  hipLaunchKernelGGL(clear_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launch attributes
hipError_t allow_dynamic_lds(const void* kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> done;  // (device, kernel) -> limit set
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  size_t& have = done[{dev, kernel}];
  if (have >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) have = bytes;
  return e;
}

}  // namespace dfl
