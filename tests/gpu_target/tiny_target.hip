// A tiny random causal target model on the GPU, for the self-contained
// speculative loop test.  It is test support, not part of the drafting
// library: the pages treat the target as an external model whose hidden
// states from several layers feed the drafter and whose logits decide
// verification ("DFlash: how block diffusion boosts NVIDIA Blackwell
// throughput", Block-diffusion architecture; "NVIDIA tests DFlash to cut LLM
// inference bottlenecks", DFlash moves token drafting to parallel compute).
//
// Pre-norm causal transformer in fp32: per layer RMSNorm -> Q/K/V with rotary
// positions -> causal GQA over the cache rows up to the row's own position ->
// O projection + residual -> RMSNorm -> SwiGLU -> down + residual; final
// RMSNorm -> LM head.  Gains are 1.
//
// Every value of a row is computed by one fixed sequence of operations that
// depends only on that row's position and the cache rows before it -- every
// reduction runs in a fixed order over a fixed thread layout, one workgroup
// per row (and head) -- so running a row alone (autoregressive decoding) or
// inside a block of rows (verification) gives bit-identical logits and
// features.  Rows of one call are processed layer by layer: a layer's K/V
// rows are all in the cache before its attention reads them.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

struct Dims {
  int vocab, hidden, n_heads, n_kv_heads, head_dim, ffn, n_layers, max_len;
  float eps, theta;
};

// Fixed-order block sum over kThreads threads (LDS tree).
__device__ float block_sum(float v, float* red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

// u = x / sqrt(mean(x^2) + eps): each thread sums its strided elements in
// order, then the tree.
__device__ void rmsnorm_row(const float* x, float* u, int H, float eps, float* red) {
  float s = 0.f;
  for (int k = threadIdx.x; k < H; k += kThreads) s += x[k] * x[k];
  const float tot = block_sum(s, red);
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  for (int k = threadIdx.x; k < H; k += kThreads) u[k] = x[k] * r;
  __syncthreads();
}

// out[o] = sum_k in[k] * W[o][k] for o = threadIdx.x, +kThreads, ... (one
// thread per output, k in order).
__device__ void matvec(const float* in, const float* W, int K, int N, float* out) {
  for (int o = threadIdx.x; o < N; o += kThreads) {
    const float* w = W + (size_t)o * K;
    float acc = 0.f;
    for (int k = 0; k < K; ++k) acc += in[k] * w[k];
    out[o] = acc;
  }
  __syncthreads();
}

__global__ void embed_kernel(const float* embed, const int32_t* tokens, int H, float* x) {
  const int r = blockIdx.x;
  const float* e = embed + (size_t)tokens[r] * H;
  for (int k = threadIdx.x; k < H; k += kThreads) x[(size_t)r * H + k] = e[k];
}

// RMSNorm -> q, k, v of one row; rotary positions on q and k; k, v into the
// layer's cache at row start + r, q into qbuf.
__global__ void qkv_kernel(Dims d, const float* x, const float* wq, const float* wk, const float* wv, float* kc,
                           float* vc, float* qbuf, int start) {
  extern __shared__ float sm[];
  const int H = d.hidden, D = d.head_dim, Nq = d.n_heads * D, Nk = d.n_kv_heads * D;
  float* red = sm;                 // kThreads
  float* u = red + kThreads;       // H
  float* q = u + H;                // Nq
  float* k = q + Nq;               // Nk
  float* v = k + Nk;               // Nk
  const int r = blockIdx.x, pos = start + r;
  rmsnorm_row(x + (size_t)r * H, u, H, d.eps, red);
  matvec(u, wq, H, Nq, q);
  matvec(u, wk, H, Nk, k);
  matvec(u, wv, H, Nk, v);
  const int half = D / 2;
  // rotate-half pairs (j, j + D/2) of every head by pos * theta^(-2j/D)
  for (int p = threadIdx.x; p < (Nq + Nk) / 2; p += kThreads) {
    const int head = p / half, j = p - head * half;
    float* z = head < d.n_heads ? q + head * D : k + (head - d.n_heads) * D;
    const double ang = (double)pos * pow((double)d.theta, -2.0 * j / (double)D);
    const float c = (float)cos(ang), s = (float)sin(ang);
    const float a = z[j], b = z[j + half];
    z[j] = a * c - b * s;
    z[j + half] = a * s + b * c;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < Nq; i += kThreads) qbuf[(size_t)r * Nq + i] = q[i];
  for (int i = threadIdx.x; i < Nk; i += kThreads) {
    kc[(size_t)pos * Nk + i] = k[i];
    vc[(size_t)pos * Nk + i] = v[i];
  }
}

// Causal attention of one (row, head) over cache rows 0 .. start + r.
__global__ void attn_kernel(Dims d, const float* qbuf, const float* kc, const float* vc, float* obuf, int start) {
  extern __shared__ float sm[];
  const int D = d.head_dim, Nq = d.n_heads * D, Nk = d.n_kv_heads * D;
  const int r = blockIdx.x, h = blockIdx.y, kvh = h / (d.n_heads / d.n_kv_heads);
  const int nk = start + r + 1;
  float* red = sm;            // kThreads
  float* p = red + kThreads;  // nk scores
  const float* q = qbuf + (size_t)r * Nq + h * D;
  const float scale = 1.0f / sqrtf((float)D);
  for (int j = threadIdx.x; j < nk; j += kThreads) {
    const float* kr = kc + (size_t)j * Nk + kvh * D;
    float s = 0.f;
    for (int i = 0; i < D; ++i) s += q[i] * kr[i];
    p[j] = s * scale;
  }
  __syncthreads();
  float m = -INFINITY;
  for (int j = threadIdx.x; j < nk; j += kThreads) m = fmaxf(m, p[j]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  m = red[0];
  __syncthreads();
  float l = 0.f;
  for (int j = threadIdx.x; j < nk; j += kThreads) {
    p[j] = expf(p[j] - m);
    l += p[j];
  }
  const float tot = block_sum(l, red);
  for (int i = threadIdx.x; i < D; i += kThreads) {
    float acc = 0.f;
    for (int j = 0; j < nk; ++j) acc += p[j] * vc[(size_t)j * Nk + kvh * D + i];
    obuf[(size_t)r * Nq + h * D + i] = acc / tot;
  }
}

// x += o W_o^T; u = RMSNorm(x); x += (SiLU(u W_g^T) * (u W_u^T)) W_d^T; the
// features of a fused layer.
__global__ void mlp_kernel(Dims d, float* x, const float* obuf, const float* wo, const float* wg, const float* wu,
                           const float* wdn, float* feat) {
  extern __shared__ float sm[];
  const int H = d.hidden, F = d.ffn, Nq = d.n_heads * d.head_dim;
  float* red = sm;           // kThreads
  float* xr = red + kThreads;  // H
  float* t = xr + H;         // max(H, F)
  float* g = t + (H > F ? H : F);  // F
  float* up = g + F;         // F
  const int r = blockIdx.x;
  float* xg = x + (size_t)r * H;
  matvec(obuf + (size_t)r * Nq, wo, Nq, H, t);
  for (int k = threadIdx.x; k < H; k += kThreads) xr[k] = xg[k] + t[k];
  __syncthreads();
  rmsnorm_row(xr, t, H, d.eps, red);
  matvec(t, wg, H, F, g);
  matvec(t, wu, H, F, up);
  for (int k = threadIdx.x; k < F; k += kThreads) g[k] = g[k] / (1.0f + expf(-g[k])) * up[k];
  __syncthreads();
  matvec(g, wdn, F, H, t);
  for (int k = threadIdx.x; k < H; k += kThreads) {
    const float v = xr[k] + t[k];
    xg[k] = v;
    if (feat) feat[(size_t)r * H + k] = v;
  }
}

__global__ void lmhead_kernel(Dims d, const float* x, const float* wlm, float* logits) {
  extern __shared__ float sm[];
  const int H = d.hidden;
  float* red = sm;
  float* u = red + kThreads;
  const int r = blockIdx.x;
  rmsnorm_row(x + (size_t)r * H, u, H, d.eps, red);
  matvec(u, wlm, H, d.vocab, logits + (size_t)r * d.vocab);
}

}  // namespace

extern "C" {

// One forward of n rows at positions start .. start+n-1 (appending their K/V
// to the per-layer caches kc[l], vc[l], each [max_len, Hkv*D] fp32).
//  w: host array of device pointers: embed, then per layer wq, wk, wv, wo, wg,
//     wu, wd, then w_lm (2 + 7 * n_layers entries), all fp32 [out, in].
//  feat_layer: host array of n_layers ints, the output slot of a fused layer's
//     features or -1; feats: device [n_feat][n][H].
//  work: device scratch of at least n * (2 * H + 2 * Nq) floats.
// Returns 0, or -1 on a bad argument, or the HIP error of a failed launch.
int tt_forward(const int* dims_i, const float* dims_f, const void* const* w, float* const* kc, float* const* vc,
               int start, const int32_t* tokens, int n, float* logits, const int* feat_layer, float* feats,
               float* work, void* stream) {
  Dims d{dims_i[0], dims_i[1], dims_i[2], dims_i[3], dims_i[4], dims_i[5], dims_i[6], dims_i[7],
         dims_f[0], dims_f[1]};
  if (n <= 0 || start < 0 || start + n > d.max_len || !w || !tokens || !logits || !work) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = d.hidden, Nq = d.n_heads * d.head_dim, Nk = d.n_kv_heads * d.head_dim, F = d.ffn;
  float* x = work;
  float* qbuf = x + (size_t)n * H;
  float* obuf = qbuf + (size_t)n * Nq;
  hipLaunchKernelGGL(embed_kernel, dim3(n), dim3(kThreads), 0, s, (const float*)w[0], tokens, H, x);
  for (int l = 0; l < d.n_layers; ++l) {
    const float* const* lw = reinterpret_cast<const float* const*>(w + 1 + 7 * l);
    const size_t qkv_lds = (size_t)(kThreads + H + Nq + 2 * Nk) * 4;
    hipLaunchKernelGGL(qkv_kernel, dim3(n), dim3(kThreads), qkv_lds, s, d, x, lw[0], lw[1], lw[2], kc[l], vc[l],
                       qbuf, start);
    const size_t attn_lds = (size_t)(kThreads + start + n) * 4;
    hipLaunchKernelGGL(attn_kernel, dim3(n, d.n_heads), dim3(kThreads), attn_lds, s, d, qbuf, kc[l], vc[l], obuf,
                       start);
    const size_t mlp_lds = (size_t)(kThreads + H + (H > F ? H : F) + 2 * F) * 4;
    float* feat = feat_layer[l] >= 0 ? feats + (size_t)feat_layer[l] * n * H : nullptr;
    hipLaunchKernelGGL(mlp_kernel, dim3(n), dim3(kThreads), mlp_lds, s, d, x, obuf, lw[3], lw[4], lw[5], lw[6], feat);
  }
  const size_t lm_lds = (size_t)(kThreads + H) * 4;
  hipLaunchKernelGGL(lmhead_kernel, dim3(n), dim3(kThreads), lm_lds, s, d, x, (const float*)w[1 + 7 * d.n_layers],
                     logits);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
