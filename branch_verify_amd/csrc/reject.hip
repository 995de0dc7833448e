// Verification of drafted trays by rejection sampling, and serving the
// prepared tray that matches the verified prefix.
//
// D3D explainer ("D3D diffusion drafter -- Asynchronous speculative
// decoding"): the target verifies a drafted block by rejection sampling with
// the proposal probabilities, which keeps the target's distribution; trays
// prepared for each plausible rejection point are served on a match.
//
// reject_chunk_kernel + reject_accept_kernel: every (tray, position) row of
// target logits is cut into chunks (one workgroup each: chunk max, first
// argmax, fast exp sum with its bound), then one wave per row merges them.
// T > 0: z = fl32(l * invT), M = max z; at a drafted position the acceptance
// test u * q(x) < p(x), p(x) = exp(z_x - M) / S, is taken on the fast S with
// its proven error bound, and on the exact fp64 S only when the bound
// straddles the threshold.  T = 0: acceptance iff the drafted token is the
// first argmax.
// reject_emit_sum_kernel, reject_sample_kernel: T > 0 only.  Each tray's
// emitting row (its first rejection, else the bonus row) is cut into chunks:
// exact fp64 partial denominators, then each chunk's best Gumbel-max key
// over the residual ln(p - q) + g (or the bonus key z + g), all in fp64.
// reject_finalize_kernel: one wave per tray merges the chunks.
// match_trays_kernel: one wave finds the lowest prepared tray matching.
#include "common.h"
#include "internal.h"
#include "noise.h"

namespace sfv {
namespace {

constexpr int kThreads = 256;
constexpr uint64_t kStreamAccept = 1, kStreamSample = 2;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct RejectArgs {
  const float* logits;    // [n][B+1][V]
  const float* q;         // [n][B][V]
  const int32_t* tokens;  // [n][B]
  int n, B, V;
  bool noisy;
  float inv_t;
  uint64_t seed, step0;
  int64_t pos0;
  int S, C;               // chunks per emitting row, ids per chunk
  RejectWs ws;
  int32_t* n_accept;
  int32_t* next_token;
};

__device__ __forceinline__ bool better_d(double v, int i, double bv, int bi) {
  return (v > bv) | ((v == bv) & (i < bi));
}

__device__ __forceinline__ void block_reduce_max_f(float& v, int& i, float* sv, int* si) {
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, kWave);
    const int oi = __shfl_xor(i, o, kWave);
    const bool take = (ov > v) | ((ov == v) & (oi < i));
    v = take ? ov : v;
    i = take ? oi : i;
  }
  if (lane == 0) {
    sv[wave] = v;
    si[wave] = i;
  }
  __syncthreads();
  v = sv[0];
  i = si[0];
  for (int w = 1; w < kThreads / kWave; ++w) {
    const bool take = (sv[w] > v) | ((sv[w] == v) & (si[w] < i));
    v = take ? sv[w] : v;
    i = take ? si[w] : i;
  }
  __syncthreads();
}

// First rejected position of tray j (B if every drafted token passes).
__device__ __forceinline__ int first_reject(const RejectArgs& a, int j) {
  int r = a.B;
  for (int t = a.B - 1; t >= 0; --t)
    if (!a.ws.accept[j * (a.B + 1) + t]) r = t;
  return r;
}

constexpr int kUnroll = 4;

// Per (row, chunk): the chunk's max of z (T > 0: fl32(l * invT); T = 0: l)
// with its first index, and (T > 0) the fast sum of exp(z - chunk max) with
// its error bound.  Fast terms: d = fl32(z - m) and c = fl32(d * log2 e)
// carry a relative exponent error below 3 * 2^-24 |c|; hardware exp2 is
// within 2^-22 on [-126, 0] (certified by the self-check); terms flushed
// below 2^-126 are covered by an absolute 2^-126 each.
__global__ __launch_bounds__(kThreads) void reject_chunk_kernel(RejectArgs a) {
  __shared__ float s_v[kThreads / kWave];
  __shared__ int s_i[kThreads / kWave];
  __shared__ double s_d[kThreads / kWave], s_e[kThreads / kWave];
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int row = blockIdx.x / a.S, sc = blockIdx.x % a.S;
  const float* l = a.logits + (size_t)row * a.V;
  const int c0 = sc * a.C, c1 = min(a.V, c0 + a.C);
  const float scale = a.noisy ? a.inv_t : 1.f;

  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int v0 = c0 + t; v0 < c1; v0 += kThreads * kUnroll) {
    float x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = l[min(v0 + u * kThreads, c1 - 1)];  // loads unconditional
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kThreads;
      const float z = x[u] * scale;
      const bool take = (v < c1) & ((z > bv) | ((z == bv) & (v < bi)));
      bv = take ? z : bv;
      bi = take ? v : bi;
    }
  }
  block_reduce_max_f(bv, bi, s_v, s_i);
  const int slot = row * a.S + sc;
  if (t == 0) {
    a.ws.chunk_max[slot] = bv;
    a.ws.chunk_arg[slot] = bi;
  }
  if (!a.noisy) return;
  const float m = bv;
  const float log2e = 1.4426950408889634f;
  double sum = 0.0, err = 0.0;
  for (int v0 = c0 + t; v0 < c1; v0 += kThreads * kUnroll) {
    float x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = l[min(v0 + u * kThreads, c1 - 1)];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float c = (x[u] * a.inv_t - m) * log2e;
      const double tv = v0 + u * kThreads < c1 ? (double)__builtin_amdgcn_exp2f(c) : 0.0;
      sum += tv;
      err += tv * (2.4e-7 + 1.8e-7 * (double)fabsf(c));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sum += __shfl_xor(sum, o, kWave);
    err += __shfl_xor(err, o, kWave);
  }
  if (lane == 0) {
    s_d[wave] = sum;
    s_e[wave] = err;
  }
  __syncthreads();
  if (t == 0) {
    a.ws.chunk_sum_f[slot] = (s_d[0] + s_d[1]) + (s_d[2] + s_d[3]);
    a.ws.chunk_err[slot] = (s_e[0] + s_e[1]) + (s_e[2] + s_e[3]);
  }
}

// Per row: the row's max and first argmax from its chunks; at a drafted
// position the acceptance test u * q(x) < exp(z_x - M) / S, on the fast S
// (chunk sums rescaled to M by hardware exp2, bound carried) when the bound
// decides it, else on the exact fp64 S.  One wave.
__global__ __launch_bounds__(kWave) void reject_accept_kernel(RejectArgs a) {
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const int j = row / (a.B + 1), pos = row % (a.B + 1);
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int c = lane; c < a.S; c += kWave) {
    const float v = a.ws.chunk_max[row * a.S + c];
    const int i = a.ws.chunk_arg[row * a.S + c];
    const bool take = (v > bv) | ((v == bv) & (i < bi));
    bv = take ? v : bv;
    bi = take ? i : bi;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, kWave);
    const int oi = __shfl_xor(bi, o, kWave);
    const bool take = (ov > bv) | ((ov == bv) & (oi < bi));
    bv = take ? ov : bv;
    bi = take ? oi : bi;
  }
  const float M = bv;
  if (lane == 0) {
    a.ws.row_max[row] = M;
    a.ws.row_arg[row] = bi;
  }
  if (pos == a.B) return;  // the bonus row needs only its max and argmax
  const int x = min(max(a.tokens[j * a.B + pos], 0), a.V - 1);  // tokens are in [0, V)
  if (!a.noisy) {
    if (lane == 0) a.ws.accept[row] = x == bi;
    return;
  }
  const float log2e = 1.4426950408889634f;
  double S = 0.0, E = 0.0;
  for (int c = lane; c < a.S; c += kWave) {
    const float arg = (a.ws.chunk_max[row * a.S + c] - M) * log2e;
    const double r = (double)__builtin_amdgcn_exp2f(arg);
    const double eps = 2.4e-7 + 1.8e-7 * (double)fabsf(arg);
    const double sc = a.ws.chunk_sum_f[row * a.S + c];
    S += sc * r;
    E += (a.ws.chunk_err[row * a.S + c] + sc * eps) * r;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    S += __shfl_xor(S, o, kWave);
    E += __shfl_xor(E, o, kWave);
  }
  E = E * 1.01 + (double)a.V * 1.2e-38 + S * 1e-10;
  const float* l = a.logits + (size_t)row * a.V;
  const double ex = exp((double)(l[x] * a.inv_t) - (double)M);
  const unsigned w = noise_word(a.seed, a.step0 + (uint64_t)j, (uint64_t)(a.pos0 + pos), 0, kStreamAccept);
  const double u = ((double)w + 0.5) * 2.3283064365386962890625e-10;
  const double uq = u * (double)a.q[((size_t)j * a.B + pos) * a.V + x];
  int acc;
  if (uq * (S + E) < ex * (1.0 - 1e-15)) {
    acc = 1;
  } else if (uq * (S - E) > ex * (1.0 + 1e-15)) {
    acc = 0;
  } else {  // the bound straddles the threshold: the exact fp64 sum decides
    double exact = 0.0;
    for (int v = lane; v < a.V; v += kWave) exact += exp((double)(l[v] * a.inv_t) - (double)M);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) exact += __shfl_xor(exact, o, kWave);
    acc = uq < ex / exact;
  }
  if (lane == 0) a.ws.accept[row] = acc;
}

// Exact fp64 softmax denominators of each tray's emitting row when it emits
// from the residual: partial sums per chunk (summed in chunk order by the
// sampler).
__global__ __launch_bounds__(kThreads) void reject_emit_sum_kernel(RejectArgs a) {
  __shared__ double s_d[kThreads / kWave];
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int j = blockIdx.x / a.S, sc = blockIdx.x % a.S;
  const int r = first_reject(a, j);
  if (r == a.B) return;
  const int row = j * (a.B + 1) + r;
  const float* l = a.logits + (size_t)row * a.V;
  const float M = a.ws.row_max[row];
  const int c0 = sc * a.C, c1 = min(a.V, c0 + a.C);
  double sum = 0.0;
  for (int v = c0 + t; v < c1; v += kThreads) sum += exp((double)(l[v] * a.inv_t) - (double)M);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
  if (lane == 0) s_d[wave] = sum;
  __syncthreads();
  if (t == 0) a.ws.chunk_sum[j * a.S + sc] = (s_d[0] + s_d[1]) + (s_d[2] + s_d[3]);
}

__global__ __launch_bounds__(kThreads) void reject_sample_kernel(RejectArgs a) {
  __shared__ double s_k[kThreads / kWave];
  __shared__ int s_i[kThreads / kWave];
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int j = blockIdx.x / a.S, sc = blockIdx.x % a.S;
  const int r = first_reject(a, j);
  const int row = j * (a.B + 1) + r;
  const float* l = a.logits + (size_t)row * a.V;
  const float* qr = a.q + ((size_t)j * a.B + min(r, a.B - 1)) * a.V;
  const bool residual = r < a.B;
  const float M = a.ws.row_max[row];
  double S = 0.0;
  if (residual)
    for (int c = 0; c < a.S; ++c) S += a.ws.chunk_sum[j * a.S + c];
  const uint64_t step = a.step0 + (uint64_t)j, posn = (uint64_t)(a.pos0 + r);
  const int c0 = sc * a.C, c1 = min(a.V, c0 + a.C);
  double bk = -INFINITY;
  int bi = 0x7FFFFFFF;
  // each thread takes runs of 8 consecutive ids (one Philox call per run)
  for (int base = c0 + 8 * t; base < c1; base += 8 * kThreads) {
    unsigned w[8];
    noise_block(a.seed, step, posn, (uint64_t)(base >> 3), w, kStreamSample);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int v = base + e;
      if (v >= c1) continue;
      const double z = (double)(l[v] * a.inv_t);
      double key;
      if (residual) {
        const double res = exp(z - (double)M) / S - (double)qr[v];
        if (!(res > 0.0)) continue;
        key = log(res);
      } else {
        key = z;
      }
      key += gumbel_exact_f64(w[e]);
      const bool take = better_d(key, v, bk, bi);
      bk = take ? key : bk;
      bi = take ? v : bi;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double ok = __shfl_xor(bk, o, kWave);
    const int oi = __shfl_xor(bi, o, kWave);
    const bool take = better_d(ok, oi, bk, bi);
    bk = take ? ok : bk;
    bi = take ? oi : bi;
  }
  if (lane == 0) {
    s_k[wave] = bk;
    s_i[wave] = bi;
  }
  __syncthreads();
  if (t == 0) {
    for (int w2 = 1; w2 < kThreads / kWave; ++w2) {
      const bool take = better_d(s_k[w2], s_i[w2], bk, bi);
      bk = take ? s_k[w2] : bk;
      bi = take ? s_i[w2] : bi;
    }
    a.ws.chunk_key[j * a.S + sc] = bk;
    a.ws.chunk_id[j * a.S + sc] = bi;
  }
}

__global__ __launch_bounds__(kWave) void reject_finalize_kernel(RejectArgs a) {
  const int lane = threadIdx.x;
  const int j = blockIdx.x;
  const int r = first_reject(a, j);
  int tok;
  if (!a.noisy) {
    tok = a.ws.row_arg[j * (a.B + 1) + r];
  } else {
    // (an empty residual, p <= q everywhere by rounding, emits the first argmax of z)
    double bk = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int c = lane; c < a.S; c += kWave) {
      const double k = a.ws.chunk_key[j * a.S + c];
      const int i = a.ws.chunk_id[j * a.S + c];
      const bool take = better_d(k, i, bk, bi);
      bk = take ? k : bk;
      bi = take ? i : bi;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ok = __shfl_xor(bk, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      const bool take = better_d(ok, oi, bk, bi);
      bk = take ? ok : bk;
      bi = take ? oi : bi;
    }
    tok = bi == 0x7FFFFFFF ? a.ws.row_arg[j * (a.B + 1) + r] : bi;
  }
  if (lane == 0) {
    a.n_accept[j] = r;
    a.next_token[j] = tok;
  }
}

__global__ __launch_bounds__(kWave) void match_trays_kernel(const int32_t* n_accept, const int32_t* next_token,
                                                            int verified, const int32_t* tray_k,
                                                            const int32_t* tray_alt, int n_prepared,
                                                            int32_t* served) {
  const int lane = threadIdx.x;
  const int a0 = n_accept[verified], c0 = next_token[verified];
  int found = -1;
  for (int b0 = 0; b0 < n_prepared; b0 += kWave) {
    const int k = b0 + lane;
    const bool hit = k < n_prepared && tray_k[k] == a0 && tray_alt[k] == c0;
    const unsigned long long bal = __ballot(hit);
    if (bal != 0ull) {
      found = b0 + __ffsll((long long)bal) - 1;
      break;
    }
  }
  if (lane == 0) served[0] = found;
}

}  // namespace

RejectPlan reject_plan(int n, int B, int V) {
  RejectPlan pl;
  int S = (V + kRejectChunkTarget - 1) / kRejectChunkTarget;
  S = S < 1 ? 1 : (S > kMaxRejectChunks ? kMaxRejectChunks : S);
  int C = (V + S - 1) / S;
  C = (C + 7) / 8 * 8;  // runs of 8 ids stay in one chunk
  S = (V + C - 1) / C;
  pl.S = S;
  pl.C = C;
  const size_t rows = (size_t)n * (B + 1);
  pl.ws_bytes = align256(rows * sizeof(float)) + align256(rows * sizeof(int)) + align256(rows * sizeof(int)) +
                align256((size_t)n * S * sizeof(double)) + align256((size_t)n * S * sizeof(double)) +
                align256((size_t)n * S * sizeof(int)) + align256(rows * S * sizeof(float)) +
                align256(rows * S * sizeof(int)) + 2 * align256(rows * S * sizeof(double));
  return pl;
}

RejectWs reject_ws(void* base, int n, int B, const RejectPlan& plan) {
  char* p = (char*)base;
  const size_t rows = (size_t)n * (B + 1);
  RejectWs ws;
  ws.row_max = (float*)p;
  p += align256(rows * sizeof(float));
  ws.row_arg = (int*)p;
  p += align256(rows * sizeof(int));
  ws.accept = (int*)p;
  p += align256(rows * sizeof(int));
  ws.chunk_sum = (double*)p;
  p += align256((size_t)n * plan.S * sizeof(double));
  ws.chunk_key = (double*)p;
  p += align256((size_t)n * plan.S * sizeof(double));
  ws.chunk_id = (int*)p;
  p += align256((size_t)n * plan.S * sizeof(int));
  ws.chunk_max = (float*)p;
  p += align256(rows * plan.S * sizeof(float));
  ws.chunk_arg = (int*)p;
  p += align256(rows * plan.S * sizeof(int));
  ws.chunk_sum_f = (double*)p;
  p += align256(rows * plan.S * sizeof(double));
  ws.chunk_err = (double*)p;
  return ws;
}

hipError_t launch_reject(const float* logits, const float* q, const int32_t* tokens, int n, int B, int V,
                         float temperature, uint64_t seed, uint64_t step0, int64_t pos0, int32_t* n_accept,
                         int32_t* next_token, void* ws, const RejectPlan& plan, hipStream_t stream) {
  RejectArgs a;
  a.logits = logits;
  a.q = q;
  a.tokens = tokens;
  a.n = n;
  a.B = B;
  a.V = V;
  a.noisy = temperature != 0.f;
  a.inv_t = a.noisy ? 1.0f / temperature : 1.f;
  a.seed = seed;
  a.step0 = step0;
  a.pos0 = pos0;
  a.S = plan.S;
  a.C = plan.C;
  a.ws = reject_ws(ws, n, B, plan);
  a.n_accept = n_accept;
  a.next_token = next_token;
  hipLaunchKernelGGL(reject_chunk_kernel, dim3(n * (B + 1) * plan.S), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reject_accept_kernel, dim3(n * (B + 1)), dim3(kWave), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.noisy) {
    hipLaunchKernelGGL(reject_emit_sum_kernel, dim3(n * plan.S), dim3(kThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(reject_sample_kernel, dim3(n * plan.S), dim3(kThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(reject_finalize_kernel, dim3(n), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_match_trays(const int32_t* n_accept, const int32_t* next_token, int verified,
                              const int32_t* tray_k, const int32_t* tray_alt, int n_prepared, int32_t* served,
                              hipStream_t stream) {
  hipLaunchKernelGGL(match_trays_kernel, dim3(1), dim3(kWave), 0, stream, n_accept, next_token, verified, tray_k,
                     tray_alt, n_prepared, served);
  return hipGetLastError();
}

}  // namespace sfv
