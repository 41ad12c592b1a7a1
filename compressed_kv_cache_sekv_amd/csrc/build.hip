// Prefill index build of the SeKV cache, gfx950.
//
// SeKV article (aitrends.kr/articles/75020):
//  * section 방법론 (Method): token surprisal H_t marks span boundaries where
//    it exceeds mu + alpha*sigma, the boundary tokens are kept as anchors;
//    anchors and very short spans stay raw on the GPU; per span the GPU keeps
//    a summary key projected to d' dims and surprisal-weighted mean key and
//    value, while the span's key and value matrices get a truncated SVD per
//    layer and head; the SVD is randomized to parallelise prefill.
//  * section 핵심 기여 (Key contributions): the summary and the mean K/V are
//    surprisal-weighted.
//  * section 기술 상세 (Technical details): the reconstruction
//    Khat_S = sum_i m_i sigma_i u_i v_i^T, so sigma_i * m_i is stored.
//
// Kernels: span_split (one workgroup per sequence), pack_raw (raw rows into the
// resident layouts), summaries (one wave per (b, l, g, span)), rsvd (one
// workgroup per (b, l, g, span, K|V) matrix).
#include "common.h"

namespace sekv {

__device__ __forceinline__ float bf(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ bf16_t to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  return (bf16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------- scans ---

// Block-wide exclusive scan of one int per thread for a 1024-thread block.
// Returns the exclusive prefix; *total receives the block total.
__device__ int scan1024(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0;
    for (int w = 0; w < 16; ++w) { const int t = s_tmp[w]; s_tmp[w] = c; c += t; }
    s_tmp[16] = c;
  }
  __syncthreads();
  const int ex = s_tmp[wave] + x - v;
  *total = s_tmp[16];
  __syncthreads();
  return ex;
}

// Fixed-order block sum of doubles (1024 threads): the result does not depend
// on scheduling.
__device__ double sum1024(double v, double* s_d) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  if ((threadIdx.x & 63) == 0) s_d[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < 16; ++w) t += s_d[w];
  __syncthreads();
  return t;
}

// ----------------------------------------------------------- span split ---
// mu and sigma: mean and population std of the sequence's surprisal in fp64;
// anchors: H_t > mu + alpha_sp*sigma (strict); spans: maximal anchor-free runs
// of at least l_min tokens; raw: anchors and the tokens of shorter runs.
__global__ __launch_bounds__(1024) void span_split_kernel(const SplitArgs a) {
  __shared__ double s_d[16];
  __shared__ int s_tmp[17];
  const int b = blockIdx.x, T = a.T, tid = threadIdx.x;
  const float* H = a.H + (int64_t)b * T;
  double acc = 0.0;
  for (int i = tid; i < T; i += 1024) acc += (double)H[i];
  const double mu = sum1024(acc, s_d) / (double)T;
  acc = 0.0;
  for (int i = tid; i < T; i += 1024) {
    const double dv = (double)H[i] - mu;
    acc += dv * dv;
  }
  const double sigma = sqrt(sum1024(acc, s_d) / (double)T);
  const double thr = mu + a.alpha_sp * sigma;
  auto anc = [&](int i) -> bool { return (double)H[i] > thr; };

  const int C = (T + 1023) / 1024;
  const int t0 = min(T, tid * C), t1 = min(T, t0 + C);
  int ns = 0, ne = 0;
  for (int i = t0; i < t1; ++i) {
    if (anc(i)) continue;
    ns += (i == 0 || anc(i - 1));
    ne += (i == T - 1 || anc(i + 1));
  }
  int nruns, nruns2;
  const int bs = scan1024(ns, s_tmp, &nruns);
  const int be = scan1024(ne, s_tmp, &nruns2);
  int32_t* starts = a.scratch + (int64_t)b * 2 * (T / 2 + 2);
  int32_t* ends = starts + (T / 2 + 2);
  {
    int ks = bs, ke = be;
    for (int i = t0; i < t1; ++i) {
      if (anc(i)) continue;
      if (i == 0 || anc(i - 1)) starts[ks++] = i;
      if (i == T - 1 || anc(i + 1)) ends[ke++] = i;
    }
  }
  __syncthreads();
  // compressed runs -> span table, in run order
  const int Cr = (nruns + 1023) / 1024;
  const int r0 = min(nruns, tid * Cr), r1 = min(nruns, r0 + Cr);
  int nc = 0;
  for (int r = r0; r < r1; ++r) nc += (ends[r] - starts[r] + 1 >= a.l_min);
  int n_spans;
  int sb = scan1024(nc, s_tmp, &n_spans);
  int32_t* sst = a.span_start + (int64_t)b * a.S_max;
  int32_t* sln = a.span_len + (int64_t)b * a.S_max;
  float* slg = a.span_logn + (int64_t)b * a.S_max;
  for (int r = r0; r < r1; ++r) {
    const int len = ends[r] - starts[r] + 1;
    if (len >= a.l_min) {
      sst[sb] = starts[r];
      sln[sb] = len;
      slg[sb] = logf((float)len);
      ++sb;
    }
  }
  // raw tokens: anchors and members of short runs, in position order
  int nraw = 0;
  {
    int run = bs - 1;  // the last run that started before t0 (bs starts precede the chunk)
    for (int i = t0; i < t1; ++i) {
      if (anc(i)) { ++nraw; continue; }
      if (i == 0 || anc(i - 1)) ++run;
      nraw += (ends[run] - starts[run] + 1 < a.l_min);
    }
  }
  int n_raw;
  int rb = scan1024(nraw, s_tmp, &n_raw);
  int32_t* rp = a.raw_pos + (int64_t)b * T;
  {
    int run = bs - 1;
    for (int i = t0; i < t1; ++i) {
      if (anc(i)) { rp[rb++] = i; continue; }
      if (i == 0 || anc(i - 1)) ++run;
      if (ends[run] - starts[run] + 1 < a.l_min) rp[rb++] = i;
    }
  }
  if (tid == 0) {
    a.counts[2 * b] = n_spans;
    a.counts[2 * b + 1] = n_raw;
  }
}

hipError_t launch_span_split(const SplitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(span_split_kernel, dim3(a.B), dim3(1024), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- raw rows ---
// grid (ceil(max_raw * D/8 / 256), B, L * Hkv): one 16-byte chunk per thread.
__global__ __launch_bounds__(256) void pack_raw_kernel(const PackArgs a) {
  const int b = blockIdx.y, lg = blockIdx.z, D = a.D;
  const BMeta bm = a.meta[b];
  const int cpr = D >> 3;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int row = (int)(gid / cpr), c = (int)(gid - (int64_t)row * cpr);
  if (row >= bm.n_raw) return;
  const int pos = a.raw_pos[bm.raw_base + row];
  const int64_t src = (((int64_t)b * a.L * a.Hkv + lg) * a.T + pos) * D + 8 * c;
  const int64_t dst = bm.res_base + (int64_t)lg * bm.n_res_pad * D;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  *(u32x4*)(a.kres + dst + krow_off(row, 8 * c, D)) = *(const u32x4*)(a.K + src);
  const bf16_t* vs = a.V + src;
#pragma unroll
  for (int e = 0; e < 8; ++e) a.vres[dst + vrow_off(row, 8 * c + e, D)] = vs[e];
}

hipError_t launch_pack_raw(const PackArgs& a, hipStream_t st) {
  const int64_t chunks = (int64_t)a.max_raw * (a.D / 8);
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_raw_kernel, dim3((unsigned)((chunks + 255) / 256), a.B, a.L * a.Hkv),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ summaries ---
// Correctly rounded fp64 -> bf16 (round to nearest even): round to odd into
// fp32 first (24 >= 8 + 2 bits), then round to nearest even; this composition
// equals direct rounding (no double-rounding error).
__device__ __forceinline__ bf16_t f64_to_bf16(double x) {
  float f = __double2float_rz(x);
  uint32_t u = __float_as_uint(f);
  if ((double)f != x) u |= 1u;
  return (bf16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// One wave per (b, l, g, span): surprisal-weighted mean key/value in fp64
// (uniform weights if the weights sum to zero), stored as the span's pseudo
// row in bf16, and s^(l,h) = W^(l,h) kbar in fp64 from the unrounded kbar,
// stored fp32, for the G query heads of KV head g.  grid (ceil(max_spans/4),
// B, L*Hkv).
__global__ __launch_bounds__(256) void summaries_kernel(const PackArgs a) {
  __shared__ double s_k[4][128];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int S = blockIdx.x * 4 + wave, b = blockIdx.y, lg = blockIdx.z;
  const int l = lg / a.Hkv, g = lg - l * a.Hkv, D = a.D;
  const BMeta bm = a.meta[b];
  const bool live = S < bm.n_spans;
  if (live) {
    const int start = a.span_start[bm.span_base + S], n = a.span_len[bm.span_base + S];
    const float* H = a.H + (int64_t)b * a.T + start;
    const int64_t src = (((int64_t)b * a.L * a.Hkv + lg) * a.T + start) * D;
    const bf16_t* K = a.K + src;
    const bf16_t* V = a.V + src;
    const int per = D >> 6;  // dims per lane: 1 (d=64) or 2 (d=128)
    double ak[2] = {0.0, 0.0}, av[2] = {0.0, 0.0}, ws = 0.0;
    for (int t = 0; t < n; ++t) {
      const double w = (double)H[t];
      ws += w;
      for (int e = 0; e < per; ++e) {
        ak[e] += w * (double)bf(K[(int64_t)t * D + per * lane + e]);
        av[e] += w * (double)bf(V[(int64_t)t * D + per * lane + e]);
      }
    }
    if (ws == 0.0) {
      ws = (double)n;
      ak[0] = ak[1] = av[0] = av[1] = 0.0;
      for (int t = 0; t < n; ++t)
        for (int e = 0; e < per; ++e) {
          ak[e] += (double)bf(K[(int64_t)t * D + per * lane + e]);
          av[e] += (double)bf(V[(int64_t)t * D + per * lane + e]);
        }
    }
    const int64_t dst = bm.res_base + (int64_t)lg * bm.n_res_pad * D;
    const int prow = bm.n_raw + S;
    for (int e = 0; e < per; ++e) {
      const int dim = per * lane + e;
      const double kb = ak[e] / ws, vb = av[e] / ws;
      s_k[wave][dim] = kb;
      a.kres[dst + krow_off(prow, dim, D)] = f64_to_bf16(kb);
      a.vres[dst + vrow_off(prow, dim, D)] = f64_to_bf16(vb);
    }
  }
  __syncthreads();
  if (!live) return;
  const int G = a.Hq / a.Hkv;
  for (int o = lane; o < G * a.dp; o += 64) {
    const int hh = g * G + o / a.dp, j = o - (o / a.dp) * a.dp;
    const float* w = a.W + (((int64_t)l * a.Hq + hh) * a.dp + j) * D;
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += (double)w[d] * s_k[wave][d];
    a.s[bm.s_base + (((int64_t)l * a.Hq + hh) * a.dp + j) * bm.s_pad + S] = (float)acc;
  }
}

hipError_t launch_summaries(const PackArgs& a, hipStream_t st) {
  if (a.max_spans == 0) return hipSuccess;
  hipLaunchKernelGGL(summaries_kernel, dim3((a.max_spans + 3) / 4, a.B, a.L * a.Hkv), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ----------------------------------------------------------------- rsvd ---
// Truncated SVD of one span matrix A (n x d, bf16) by randomized subspace
// iteration (Halko, Martinsson and Tropp, "Finding structure with randomness",
// SIAM Review 2011): with sketch width l = min(R + p, n, d), the right
// singular subspace is approximated by Z = orth((A^T A)^(q+1) Omega), each
// power step re-orthonormalised (classical Gram-Schmidt, two passes); when
// l = min(n, d) the sketch already spans A's row space and Z = orth(A^T) (or
// the identity) exactly.  Rayleigh-Ritz on A^T A within span(Z) gives V and
// sigma (cyclic Jacobi on the l x l projected matrix); U = A V Sigma^-1,
// re-orthonormalised by one Cholesky-QR pass.  fp32 throughout; A^T (A Z) is
// applied as two skinny products, never forming A^T A.
// Omega ~ N(0, 1) from Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011) keyed by the seed
// and counter (matrix id, element), through the Box-Muller transform.

__device__ __forceinline__ void philox4x32_10(uint32_t ctr[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * ctr[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * ctr[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ ctr[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ ctr[3] ^ k1;
    ctr[1] = (uint32_t)p1;
    ctr[3] = (uint32_t)p0;
    ctr[0] = n0;
    ctr[2] = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

__device__ float gaussian(uint64_t seed, uint64_t mat, uint32_t idx) {
  uint32_t c[4] = {idx, (uint32_t)mat, (uint32_t)(mat >> 32), 0x5e4bu};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  const float u1 = ((float)(c[0] >> 8) + 1.0f) * (1.0f / 16777216.0f);  // (0, 1]
  const float u2 = (float)(c[1] >> 8) * (1.0f / 16777216.0f);           // [0, 1)
  return sqrtf(-2.0f * logf(u1)) * cosf(6.283185307179586f * u2);
}

struct SvdShared {
  float* Z;    // [D][LM] orthonormal basis
  float* MZ;   // [D][LM] A^T A Z, later V
  float* Y;    // [CH][LM] chunk of A Z
  float* T;    // [LM][LM]
  float* E;    // [LM][LM] eigenvectors
  float* vec;  // [4 * LM] scratch
  int LM;
};

constexpr int CH = 32;   // rows of A per chunk of A Z

// MZ[:, :l] = A^T (A Z[:, :l]); all 256 threads.
__device__ void gram_apply(const bf16_t* A, int n, int D, int l, SvdShared& s) {
  const int LM = s.LM;
  for (int i = threadIdx.x; i < D * LM; i += 256) s.MZ[i] = 0.f;
  __syncthreads();
  for (int c0 = 0; c0 < n; c0 += CH) {
    const int rows = min(CH, n - c0);
    for (int idx = threadIdx.x; idx < rows * l; idx += 256) {
      const int i = idx / l, j = idx - i * l;
      const bf16_t* ar = A + (int64_t)(c0 + i) * D;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc += bf(ar[d]) * s.Z[d * LM + j];
      s.Y[i * LM + j] = acc;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < D * l; idx += 256) {
      const int d = idx / l, j = idx - d * l;
      float acc = 0.f;
      for (int i = 0; i < rows; ++i) acc += bf(A[(int64_t)(c0 + i) * D + d]) * s.Y[i * LM + j];
      s.MZ[d * LM + j] += acc;
    }
    __syncthreads();
  }
}

// Orthonormalise the first l columns of X (D rows, stride LM) in place by
// classical Gram-Schmidt with one re-orthogonalisation; a column whose norm
// drops below 1e-6 of its original norm is set to zero.
__device__ void orth_cols(float* X, int D, int l, int LM, float* proj) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int j = 0; j < l; ++j) {
    float n0 = 0.f;
    for (int pass = 0; pass < 2; ++pass) {
      // proj[k] = X[:,k] . X[:,j] for k < j; proj[j] = |X[:,j]|^2
      for (int k = wave; k <= j; k += 4) {
        float acc = 0.f;
        for (int d = lane; d < D; d += 64) acc += X[d * LM + k] * X[d * LM + j];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
        if (lane == 0) proj[k] = acc;
      }
      __syncthreads();
      if (pass == 0) n0 = proj[j];
      for (int d = threadIdx.x; d < D; d += 256) {
        float acc = X[d * LM + j];
        for (int k = 0; k < j; ++k) acc -= proj[k] * X[d * LM + k];
        X[d * LM + j] = acc;
      }
      __syncthreads();
    }
    float acc = 0.f;
    if (wave == 0) {
      for (int d = lane; d < D; d += 64) acc += X[d * LM + j] * X[d * LM + j];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
      if (lane == 0) proj[LM] = acc;
    }
    __syncthreads();
    const float nn = proj[LM];
    const float inv = (nn > 1e-12f * n0 && nn > 0.f) ? rsqrtf(nn) : 0.f;
    for (int d = threadIdx.x; d < D; d += 256) X[d * LM + j] *= inv;
    __syncthreads();
  }
}

// Cyclic Jacobi eigen-decomposition of the symmetric l x l matrix T (in
// place, becomes diagonal) with eigenvectors accumulated in E; rotations on
// disjoint index pairs run in parallel (round-robin ordering).
__device__ void jacobi_eig(float* T, float* E, int l, int LM, float* rot) {
  const int m = l + (l & 1);  // even player count; index l is a dummy when l is odd
  for (int i = threadIdx.x; i < l * l; i += 256) {
    const int r = i / l, c = i - r * l;
    E[r * LM + c] = (r == c) ? 1.f : 0.f;
  }
  __syncthreads();
  __shared__ int s_rot_any;
  for (int sweep = 0; sweep < 15; ++sweep) {
    if (threadIdx.x == 0) s_rot_any = 0;
    __syncthreads();
    for (int rnd = 0; rnd < m - 1; ++rnd) {
      // pair k: players idx(k) and idx(m-1-k); player 0 fixed, the rest rotate
      for (int k = threadIdx.x; k < m / 2; k += 256) {
        const int a0 = k, a1 = m - 1 - k;
        const int p = (a0 == 0) ? 0 : ((a0 - 1 + rnd) % (m - 1)) + 1;
        const int q = ((a1 - 1 + rnd) % (m - 1)) + 1;
        float c = 1.f, sn = 0.f;
        if (p < l && q < l) {
          const float apq = T[p * LM + q], app = T[p * LM + p], aqq = T[q * LM + q];
          if (fabsf(apq) > 2e-7f * sqrtf(fabsf(app * aqq)) && fabsf(apq) > 1e-30f) {
            const float th = (aqq - app) / (2.f * apq);
            const float t = (th >= 0.f ? 1.f : -1.f) / (fabsf(th) + sqrtf(1.f + th * th));
            c = rsqrtf(1.f + t * t);
            sn = t * c;
            s_rot_any = 1;
          }
        }
        rot[4 * k + 0] = c;
        rot[4 * k + 1] = sn;
        rot[4 * k + 2] = __int_as_float(p);
        rot[4 * k + 3] = __int_as_float(q);
      }
      __syncthreads();
      // rows p, q of T
      for (int idx = threadIdx.x; idx < (m / 2) * l; idx += 256) {
        const int k = idx / l, col = idx - k * l;
        const int p = __float_as_int(rot[4 * k + 2]), q = __float_as_int(rot[4 * k + 3]);
        if (p >= l || q >= l) continue;
        const float c = rot[4 * k], sn = rot[4 * k + 1];
        const float tp = T[p * LM + col], tq = T[q * LM + col];
        T[p * LM + col] = c * tp - sn * tq;
        T[q * LM + col] = sn * tp + c * tq;
      }
      __syncthreads();
      // columns p, q of T and of E
      for (int idx = threadIdx.x; idx < (m / 2) * l; idx += 256) {
        const int k = idx / l, row = idx - k * l;
        const int p = __float_as_int(rot[4 * k + 2]), q = __float_as_int(rot[4 * k + 3]);
        if (p >= l || q >= l) continue;
        const float c = rot[4 * k], sn = rot[4 * k + 1];
        const float tp = T[row * LM + p], tq = T[row * LM + q];
        T[row * LM + p] = c * tp - sn * tq;
        T[row * LM + q] = sn * tp + c * tq;
        const float ep = E[row * LM + p], eq = E[row * LM + q];
        E[row * LM + p] = c * ep - sn * eq;
        E[row * LM + q] = sn * ep + c * eq;
      }
      __syncthreads();
    }
    const int any = s_rot_any;
    __syncthreads();
    if (!any) break;
  }
}

template <int D, bool BATCHED>
__global__ __launch_bounds__(256) void rsvd_kernel(const PackArgs a) {
  extern __shared__ float lds[];
  int S = 0, b = 0, g = 0, which = 0, n, l_layer = a.layer;
  const bf16_t* A;
  uint64_t mat;
  BMeta bm{};
  if (BATCHED) {
    mat = blockIdx.x;
    A = a.A + a.mat_row_off[mat];
    n = a.mat_rows[mat];
  } else {
    S = blockIdx.x; b = blockIdx.y; g = blockIdx.z >> 1; which = blockIdx.z & 1;
    bm = a.meta[b];
    if (S >= bm.n_spans) return;
    const int start = a.span_start[bm.span_base + S];
    n = a.span_len[bm.span_base + S];
    A = (which ? a.V : a.K) + (((int64_t)b * a.L * a.Hkv + (int64_t)l_layer * a.Hkv + g) * a.T + start) * D;
    mat = ((((uint64_t)b * a.L + l_layer) * a.Hkv + g) * 2 + which) * (uint64_t)a.S_max + S;
  }
  const int R = a.R;
  const int LM = R + a.oversample;
  SvdShared sh;
  sh.LM = LM;
  sh.Z = lds;
  sh.MZ = sh.Z + D * LM;
  sh.Y = sh.MZ + D * LM;
  sh.T = sh.Y + CH * LM;
  sh.E = sh.T + LM * LM;
  sh.vec = sh.E + LM * LM;
  float* rot = sh.vec + 2 * LM + 4;  // 4 * (LM/2 + 1) floats
  __shared__ int s_perm[128];
  __shared__ float s_sig[128];
  __shared__ int s_r;
  const int lw = min(LM, min(n, D));

  // ---- basis Z of the (approximate) dominant right singular subspace
  if (lw == min(n, D)) {
    for (int i = threadIdx.x; i < D * lw; i += 256) {
      const int d = i / lw, j = i - d * lw;
      sh.Z[d * LM + j] = (n <= D) ? bf(A[(int64_t)j * D + d]) : (d == j ? 1.f : 0.f);
    }
    __syncthreads();
    if (n <= D) orth_cols(sh.Z, D, lw, LM, sh.vec);
  } else {
    for (int i = threadIdx.x; i < D * lw; i += 256) {
      const int d = i / lw, j = i - d * lw;
      sh.Z[d * LM + j] = gaussian(a.seed, mat, (uint32_t)(d * lw + j));
    }
    __syncthreads();
    for (int it = 0; it <= a.power_iters; ++it) {
      gram_apply(A, n, D, lw, sh);
      for (int i = threadIdx.x; i < D * LM; i += 256) sh.Z[i] = sh.MZ[i];
      __syncthreads();
      orth_cols(sh.Z, D, lw, LM, sh.vec);
    }
  }
  // ---- Rayleigh-Ritz: T = Z^T (A^T A) Z, eigen-decomposition
  gram_apply(A, n, D, lw, sh);
  for (int idx = threadIdx.x; idx < lw * lw; idx += 256) {
    const int i = idx / lw, j = idx - i * lw;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc += sh.Z[d * LM + i] * sh.MZ[d * LM + j];
    sh.E[i * LM + j] = acc;  // staging; jacobi_eig re-initialises E
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < lw * lw; idx += 256) {
    const int i = idx / lw, j = idx - i * lw;
    sh.T[i * LM + j] = 0.5f * (sh.E[i * LM + j] + sh.E[j * LM + i]);
  }
  __syncthreads();
  jacobi_eig(sh.T, sh.E, lw, LM, rot);
  // order eigenpairs by decreasing eigenvalue (ties: lower index first)
  for (int i = threadIdx.x; i < lw; i += 256) {
    const float ti = sh.T[i * LM + i];
    int rank = 0;
    for (int j = 0; j < lw; ++j) {
      const float tj = sh.T[j * LM + j];
      rank += (tj > ti) || (tj == ti && j < i);
    }
    s_perm[rank] = i;
  }
  __syncthreads();
  const int r = min(R, lw);
  if (threadIdx.x == 0) {
    const float top = sqrtf(fmaxf(sh.T[s_perm[0] * LM + s_perm[0]], 0.f));
    int re = 0;
    for (int i = 0; i < r; ++i) {
      const float sg = sqrtf(fmaxf(sh.T[s_perm[i] * LM + s_perm[i]], 0.f));
      const bool keep = sg > 1e-6f * top && sg > 0.f;
      s_sig[i] = keep ? sg : 0.f;
      re += keep;
    }
    s_r = re;  // leading kept components (eigenvalues are sorted)
  }
  __syncthreads();
  const int re = s_r;
  // V[:, i] = Z E[:, perm[i]] into MZ
  for (int idx = threadIdx.x; idx < D * re; idx += 256) {
    const int d = idx / re, i = idx - d * re;
    const int c = s_perm[i];
    float acc = 0.f;
    for (int k = 0; k < lw; ++k) acc += sh.Z[d * LM + k] * sh.E[k * LM + c];
    sh.MZ[d * LM + i] = acc;
  }
  __syncthreads();
  // Cholesky-QR of U = A V Sigma^-1: G = Sigma^-1 (A V)^T (A V) Sigma^-1 (re x re)
  {
    float* Gm = sh.T;  // reuse
    for (int i = threadIdx.x; i < re * re; i += 256) Gm[(i / re) * LM + (i % re)] = 0.f;
    __syncthreads();
    for (int c0 = 0; c0 < n; c0 += CH) {
      const int rows = min(CH, n - c0);
      for (int idx = threadIdx.x; idx < rows * re; idx += 256) {
        const int i = idx / re, j = idx - i * re;
        const bf16_t* ar = A + (int64_t)(c0 + i) * D;
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc += bf(ar[d]) * sh.MZ[d * LM + j];
        sh.Y[i * LM + j] = acc / s_sig[j];
      }
      __syncthreads();
      for (int idx = threadIdx.x; idx < re * re; idx += 256) {
        const int i = idx / re, j = idx - i * re;
        float acc = 0.f;
        for (int t = 0; t < rows; ++t) acc += sh.Y[t * LM + i] * sh.Y[t * LM + j];
        Gm[i * LM + j] += acc;
      }
      __syncthreads();
    }
    // in-place lower Cholesky (right-looking)
    for (int k = 0; k < re; ++k) {
      if (threadIdx.x == 0) Gm[k * LM + k] = sqrtf(fmaxf(Gm[k * LM + k], 1e-30f));
      __syncthreads();
      for (int i = k + 1 + threadIdx.x; i < re; i += 256) Gm[i * LM + k] /= Gm[k * LM + k];
      __syncthreads();
      for (int idx = threadIdx.x; idx < re * re; idx += 256) {
        const int i = idx / re, j = idx - i * re;
        if (j > k && i >= j) Gm[i * LM + j] -= Gm[i * LM + k] * Gm[j * LM + k];
      }
      __syncthreads();
    }
  }
  __syncthreads();
  // Vs = V Sigma^-1 L^-T, one row of V per thread (forward substitution);
  // Z is no longer needed and holds Vs
  float* Vs = sh.Z;
  for (int d = threadIdx.x; d < D; d += 256) {
    for (int i = 0; i < re; ++i) {
      float x = sh.MZ[d * LM + i] / s_sig[i];
      for (int k = 0; k < i; ++k) x -= sh.T[i * LM + k] * Vs[d * LM + k];
      Vs[d * LM + i] = x / sh.T[i * LM + i];
    }
  }
  __syncthreads();

  if (BATCHED) {
    float* Uo = a.out_U + mat * (int64_t)a.max_rows * R;
    for (int idx = threadIdx.x; idx < n * R; idx += 256) {
      const int t = idx / R, i = idx - t * R;
      float acc = 0.f;
      if (i < re) {
        const bf16_t* ar = A + (int64_t)t * D;
        for (int d = 0; d < D; ++d) acc += bf(ar[d]) * Vs[d * LM + i];
      }
      Uo[(int64_t)t * R + i] = acc;
    }
    for (int idx = threadIdx.x + n * R; idx < a.max_rows * R; idx += 256) Uo[idx] = 0.f;
    float* Vo = a.out_Vt + mat * (int64_t)R * D;
    for (int idx = threadIdx.x; idx < R * D; idx += 256) {
      const int i = idx / D, d = idx - i * D;
      Vo[idx] = (i < re) ? sh.MZ[d * LM + i] : 0.f;
    }
    for (int i = threadIdx.x; i < R; i += 256) a.out_S[mat * R + i] = (i < re) ? s_sig[i] : 0.f;
    return;
  }
  // ---- outputs into the factor blob
  const int npad = Blob::npad(n);
  uint8_t* blob = a.pool + bm.pool_base + (int64_t)g * bm.pool_lg + a.span_off[bm.span_base + S];
  // U = A Vs (n x re), bf16; columns re..R-1 stay zero (pool is cleared)
  bf16_t* Uo = (bf16_t*)(blob + (which ? Blob::off_uvt(R, D, n) : Blob::off_uk(R, D)));
  for (int idx = threadIdx.x; idx < n * re; idx += 256) {
    const int t = idx / re, i = idx - t * re;
    const bf16_t* ar = A + (int64_t)t * D;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc += bf(ar[d]) * Vs[d * LM + i];
    const int64_t o = which ? a16_off(i, t, npad) : a16_off(t, i, R);
    Uo[o] = to_bf16(acc);
  }
  // V (right factors): K -> VKt [R][D] krow layout, V -> VV [D][R] a16 layout
  bf16_t* Vo = (bf16_t*)(blob + (which ? Blob::off_vv(R, D) : Blob::off_vkt(R, D)));
  for (int idx = threadIdx.x; idx < D * re; idx += 256) {
    const int d = idx / re, i = idx - d * re;
    const int64_t o = which ? a16_off(d, i, R) : krow_off(i, d, D);
    Vo[o] = to_bf16(sh.MZ[d * LM + i]);
  }
  // sigma * m
  float* sm = (float*)(blob + (which ? Blob::off_smv(R, D) : Blob::off_smk(R, D)));
  for (int i = threadIdx.x; i < R; i += 256) {
    float m = 1.f;
    if (a.gates)
      m = a.gates[((((int64_t)b * a.L + l_layer) * a.Hkv + g) * 2 + which) * ((int64_t)a.S_max * R) +
                  (int64_t)S * R + i];
    sm[i] = (i < re) ? s_sig[i] * m : 0.f;
  }
}

size_t rsvd_lds_bytes(int D, int LM) {
  return sizeof(float) * ((size_t)2 * D * LM + (size_t)CH * LM + 2 * (size_t)LM * LM + 2 * LM + 4 +
                          4 * (LM / 2 + 2));
}

template <int D, bool BATCHED>
static hipError_t allow_lds(size_t lds) {
  return hipFuncSetAttribute((const void*)rsvd_kernel<D, BATCHED>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_rsvd(const PackArgs& a, hipStream_t st) {
  if (a.max_spans == 0) return hipSuccess;
  const int LM = a.R + a.oversample;
  const size_t lds = rsvd_lds_bytes(a.D, LM);
  if (lds > 160 * 1024 - 2048) return hipErrorInvalidValue;
  hipError_t e = (a.D == 64) ? allow_lds<64, false>(lds) : allow_lds<128, false>(lds);
  if (e != hipSuccess) return e;
  dim3 grid(a.max_spans, a.B, a.Hkv * 2);
  if (a.D == 64) {
    hipLaunchKernelGGL((rsvd_kernel<64, false>), grid, dim3(256), lds, st, a);
  } else if (a.D == 128) {
    hipLaunchKernelGGL((rsvd_kernel<128, false>), grid, dim3(256), lds, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rsvd_batched(const PackArgs& a, hipStream_t st) {
  if (a.count == 0) return hipSuccess;
  const int LM = a.R + a.oversample;
  const size_t lds = rsvd_lds_bytes(a.D, LM);
  if (lds > 160 * 1024 - 2048) return hipErrorInvalidValue;
  hipError_t e = (a.D == 64) ? allow_lds<64, true>(lds) : allow_lds<128, true>(lds);
  if (e != hipSuccess) return e;
  if (a.D == 64) {
    hipLaunchKernelGGL((rsvd_kernel<64, true>), dim3(a.count), dim3(256), lds, st, a);
  } else if (a.D == 128) {
    hipLaunchKernelGGL((rsvd_kernel<128, true>), dim3(a.count), dim3(256), lds, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sekv
