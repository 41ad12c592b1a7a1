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
//    Khat_S = sum_i m_i sigma_i u_i v_i^T, so sigma_i * m_i is stored; the
//    components are dropped at storage and transfer, and section 핵심 기여
//    (Key contributions) has the gates set each span's effective rank: a
//    component whose gate is below the build's gate_eps is not stored.
//
// Kernels: span_split (one workgroup per sequence), ranks (stored rank of
// every span factorization, which sizes the factor pool), pack_raw (raw rows
// into the resident layouts), summaries (one wave per (b, l, g, span)).  The
// truncated SVD of the spans is in rsvd.hip.
#include "common.h"

namespace sekv {

__device__ __forceinline__ float bf(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ bf16_t to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  return (bf16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------- ranks ---

// One thread per (b, l, g, span slot): the components kept of the span's K
// and V factorizations (i < min(R, n) with gate_kept), as stored ranks.  Slots
// at or past N_S(b) write 0.
__global__ __launch_bounds__(256) void rank_kernel(const RankArgs a) {
  const int nbx = (a.S_max + 255) / 256;
  const int blg = blockIdx.x / nbx;   // (b L + l) Hkv + g
  const int S = (blockIdx.x - blg * nbx) * 256 + threadIdx.x;
  const int b = blg / (a.L * a.Hkv);
  if (S >= a.S_max) return;
  uint32_t* out = a.ranks + (int64_t)blg * a.S_max + S;
  if (S >= a.counts[2 * b]) {
    *out = 0u;
    return;
  }
  const int n = a.span_len[(int64_t)b * a.S_max + S];
  const int r = min(a.R, n);
  int kept[2];
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    int c = 0;
    if (a.gates) {
      const float* m = a.gates + (((int64_t)blg * 2 + which) * a.S_max + S) * a.R;
      for (int i = 0; i < r; ++i) c += gate_kept(m[i], a.gate_eps);
    } else {
      c = gate_kept(1.f, a.gate_eps) ? r : 0;
    }
    kept[which] = stored_rank(c);
  }
  *out = (uint32_t)kept[0] | ((uint32_t)kept[1] << 16);
}

hipError_t launch_ranks(const RankArgs& a, hipStream_t st) {
  if (a.S_max < 1 || a.B * a.L * a.Hkv < 1) return hipSuccess;
  const int64_t blocks = (int64_t)((a.S_max + 255) / 256) * a.B * a.L * a.Hkv;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rank_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
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
// One 1024-thread workgroup per sequence.

// The anchor threshold mu + alpha_sp * sigma of one sequence (fixed-order sums).
__device__ double split_threshold(const float* H, int T, double alpha_sp, double* s_d) {
  double acc = 0.0;
  for (int i = threadIdx.x; i < T; i += 1024) acc += (double)H[i];
  const double mu = sum1024(acc, s_d) / (double)T;
  acc = 0.0;
  for (int i = threadIdx.x; i < T; i += 1024) {
    const double dv = (double)H[i] - mu;
    acc += dv * dv;
  }
  const double sigma = sqrt(sum1024(acc, s_d) / (double)T);
  return mu + alpha_sp * sigma;
}

// Sequences of up to kSplitBitsT tokens: the anchor test is evaluated once,
// with coalesced loads, into a bitmap in LDS (bit j of word w: token 32 w + j);
// thread t then takes whole words of tokens and forms run starts, run ends and
// raw tokens with word operations (a start: a non-anchor token at 0 or after
// an anchor; an end: a non-anchor token at T - 1 or before an anchor).
constexpr int kSplitBitsT = 262144;   // 32 KB of bitmap

__global__ __launch_bounds__(1024) void span_split_bits_kernel(const SplitArgs a) {
  extern __shared__ uint32_t s_anc[];   // [2 ceil(T / 64)]
  __shared__ double s_d[16];
  __shared__ int s_tmp[17];
  const int b = blockIdx.x, T = a.T, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* H = a.H + (int64_t)b * T;
  const double thr = split_threshold(H, T, a.alpha_sp, s_d);
  const int NW = (T + 31) >> 5, NWP = 2 * ((T + 63) >> 6);   // words used, words held
  for (int i0 = 0; i0 < T; i0 += 1024) {
    const int i = i0 + tid;
    const uint64_t bal = __ballot(i < T && (double)H[i] > thr);
    if (lane == 0 && (i0 >> 5) + 2 * wave < NWP) {
      const int w = (i0 >> 5) + 2 * wave;
      s_anc[w] = (uint32_t)bal;
      s_anc[w + 1] = (uint32_t)(bal >> 32);
    }
  }
  __syncthreads();
  // this thread's words [w0, w1)
  const int CW = (NW + 1023) / 1024;
  const int w0 = min(NW, tid * CW), w1 = min(NW, w0 + CW);
  auto valid = [&](int w) -> uint32_t {   // bits of tokens < T
    const int left = T - 32 * w;
    return left >= 32 ? 0xffffffffu : ((1u << left) - 1u);
  };
  auto starts_of = [&](int w) -> uint32_t {
    const uint32_t an = s_anc[w];
    const uint32_t prev = (w == 0) ? 1u : (s_anc[w - 1] >> 31);   // token -1 counts as an anchor
    return ~an & valid(w) & ((an << 1) | prev);
  };
  auto ends_of = [&](int w) -> uint32_t {
    const uint32_t an = s_anc[w];
    uint32_t next = (an >> 1) | ((w + 1 < NW) ? (s_anc[w + 1] << 31) : 0u);
    if (32 * w + 31 >= T - 1) next |= 1u << (T - 1 - 32 * w);   // token T counts as an anchor
    return ~an & valid(w) & next;
  };
  int ns = 0, ne = 0;
  for (int w = w0; w < w1; ++w) {
    ns += __popc(starts_of(w));
    ne += __popc(ends_of(w));
  }
  int nruns, nruns2;
  const int bs = scan1024(ns, s_tmp, &nruns);
  const int be = scan1024(ne, s_tmp, &nruns2);
  int32_t* starts = a.scratch + (int64_t)b * 2 * (T / 2 + 2);
  int32_t* ends = starts + (T / 2 + 2);
  {
    int ks = bs, ke = be;
    for (int w = w0; w < w1; ++w) {
      for (uint32_t x = starts_of(w); x; x &= x - 1) starts[ks++] = 32 * w + __ffs(x) - 1;
      for (uint32_t x = ends_of(w); x; x &= x - 1) ends[ke++] = 32 * w + __ffs(x) - 1;
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
  for (int r = r0; r < r1; ++r) {
    const int len = ends[r] - starts[r] + 1;
    if (len >= a.l_min) {
      sst[sb] = starts[r];
      sln[sb] = len;
      ++sb;
    }
  }
  // raw bits of word w: its anchors and the tokens of short runs; run is the
  // index of the last run started before the word, and moves past the word's
  // starts
  auto raw_of = [&](int w, int& run) -> uint32_t {
    const uint32_t an = s_anc[w] & valid(w);
    uint32_t raw = an, rem = ~s_anc[w] & valid(w), st = starts_of(w);
    while (rem) {
      const int nb = st ? __ffs(st) - 1 : 32;   // the next start in the word
      const uint32_t seg = (nb >= 32) ? rem : (rem & ((1u << nb) - 1u));
      if (seg && ends[run] - starts[run] + 1 < a.l_min) raw |= seg;
      rem &= ~seg;
      if (!st) break;
      ++run;
      st &= st - 1;
    }
    return raw;
  };
  int nraw = 0;
  {
    int run = bs - 1;   // the last run that started before w0
    for (int w = w0; w < w1; ++w) nraw += __popc(raw_of(w, run));
  }
  int n_raw;
  int rb = scan1024(nraw, s_tmp, &n_raw);
  int32_t* rp = a.raw_pos + (int64_t)b * T;
  {
    int run = bs - 1;
    for (int w = w0; w < w1; ++w)
      for (uint32_t x = raw_of(w, run); x; x &= x - 1) rp[rb++] = 32 * w + __ffs(x) - 1;
  }
  if (tid == 0) {
    a.counts[2 * b] = n_spans;
    a.counts[2 * b + 1] = n_raw;
  }
}

// Longer sequences: each thread walks a contiguous chunk of tokens.
__global__ __launch_bounds__(1024) void span_split_kernel(const SplitArgs a) {
  __shared__ double s_d[16];
  __shared__ int s_tmp[17];
  const int b = blockIdx.x, T = a.T, tid = threadIdx.x;
  const float* H = a.H + (int64_t)b * T;
  const double thr = split_threshold(H, T, a.alpha_sp, s_d);
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
  for (int r = r0; r < r1; ++r) {
    const int len = ends[r] - starts[r] + 1;
    if (len >= a.l_min) {
      sst[sb] = starts[r];
      sln[sb] = len;
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
  if (a.T <= kSplitBitsT) {
    const size_t lds = sizeof(uint32_t) * 2 * (size_t)((a.T + 63) / 64);
    hipLaunchKernelGGL(span_split_bits_kernel, dim3(a.B), dim3(1024), lds, st, a);
  } else {
    hipLaunchKernelGGL(span_split_kernel, dim3(a.B), dim3(1024), 0, st, a);
  }
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
//  * Means: a row of d bf16 is d / 8 lanes of 16 bytes, so one load covers
//    64 / (d / 8) rows; each lane keeps kU loads of K and of V in flight (16
//    rows a round at d = 128), accumulates its 8 dims in fp64, and the row
//    slots are summed by shuffles at the end.
//  * s: thread o takes output (head, j) for all four spans of the workgroup,
//    so each W row is read once per workgroup (16-byte loads, 8 in flight),
//    summed over d in order as before.
__global__ __launch_bounds__(256) void summaries_kernel(const PackArgs a) {
  constexpr int kU = 4;
  __shared__ double s_k[4][128];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int S0 = blockIdx.x * 4, S = S0 + wave, b = blockIdx.y, lg = blockIdx.z;
  const int l = lg / a.Hkv, g = lg - l * a.Hkv, D = a.D;
  const BMeta bm = a.meta[b];
  const int CL = D >> 3, RS = 64 / CL;   // lanes per row, rows per load
  const int c = lane % CL, rs = lane / CL;
  if (S < bm.n_spans) {
    const int start = a.span_start[bm.span_base + S], n = a.span_len[bm.span_base + S];
    const float* H = a.H + (int64_t)b * a.T + start;
    const int64_t src = (((int64_t)b * a.L * a.Hkv + lg) * a.T + start) * D + 8 * c;
    const bf16_t* K = a.K + src;
    const bf16_t* V = a.V + src;
    double ak[8], av[8], ws;
    auto accumulate = [&](bool uniform) {
      ws = 0.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) ak[e] = av[e] = 0.0;
      for (int t0 = 0; t0 < n; t0 += kU * RS) {
        uint4 kv[kU], vv[kU];
        float hv[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {   // rows past the span re-read its last row (unused)
          const int t = min(t0 + rs + u * RS, n - 1);
          kv[u] = *(const uint4*)(K + (int64_t)t * D);
          vv[u] = *(const uint4*)(V + (int64_t)t * D);
          hv[u] = H[t];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          if (t0 + rs + u * RS >= n) continue;
          const double w = uniform ? 1.0 : (double)hv[u];
          ws += w;
          const uint32_t kw[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
          const uint32_t vw[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t kb = (e & 1) ? (kw[e >> 1] & 0xffff0000u) : (kw[e >> 1] << 16);
            const uint32_t vb = (e & 1) ? (vw[e >> 1] & 0xffff0000u) : (vw[e >> 1] << 16);
            ak[e] += w * (double)__uint_as_float(kb);
            av[e] += w * (double)__uint_as_float(vb);
          }
        }
      }
      for (int o = CL; o < 64; o <<= 1) {   // sum the row slots
        ws += __shfl_xor(ws, o);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ak[e] += __shfl_xor(ak[e], o);
          av[e] += __shfl_xor(av[e], o);
        }
      }
    };
    accumulate(false);
    if (ws == 0.0) accumulate(true);   // the same in every lane
    if (rs == 0) {
      const int64_t dst = bm.res_base + (int64_t)lg * bm.n_res_pad * D;
      const int prow = bm.n_raw + S;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dim = 8 * c + e;
        const double kb = ak[e] / ws, vb = av[e] / ws;
        s_k[wave][dim] = kb;
        a.kres[dst + krow_off(prow, dim, D)] = f64_to_bf16(kb);
        a.vres[dst + vrow_off(prow, dim, D)] = f64_to_bf16(vb);
      }
    }
  }
  __syncthreads();
  const int nlive = min(4, bm.n_spans - S0);
  if (nlive <= 0) return;
  const int G = a.Hq / a.Hkv, d4 = dp_pad4(a.dp);
  for (int o = threadIdx.x; o < G * a.dp; o += 256) {
    const int hh = g * G + o / a.dp, j = o - (o / a.dp) * a.dp;
    const float4* w4 = (const float4*)(a.W + (((int64_t)l * a.Hq + hh) * a.dp + j) * D);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int q0 = 0; q0 < D / 4; q0 += 8) {
      float4 wv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) wv[u] = w4[q0 + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int d = 4 * (q0 + u);
        const float wx[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int sp = 0; sp < 4; ++sp) acc[sp] += (double)wx[e] * s_k[sp][d + e];
      }
    }
    for (int sp = 0; sp < nlive; ++sp)
      a.s[bm.s_base + ((int64_t)l * a.Hq + hh) * d4 * bm.s_pad + skey_index(S0 + sp, j, d4)] = (float)acc[sp];
  }
}

hipError_t launch_summaries(const PackArgs& a, hipStream_t st) {
  if (a.max_spans == 0) return hipSuccess;
  hipLaunchKernelGGL(summaries_kernel, dim3((a.max_spans + 3) / 4, a.B, a.L * a.Hkv), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sekv
