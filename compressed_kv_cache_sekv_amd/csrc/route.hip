// Stage 1 routing of the SeKV decode step, gfx950.
//
// SeKV article (aitrends.kr/articles/75020), section 방법론 (Method): the query
// q^(l,h) is mapped by the routing projection W^(l,h), dotted with each span's
// summary key, squashed by a sigmoid into alpha_S^(l,h) and compared with the
// per-(layer, head) threshold tau^(l,h) to decide z_S^(l,h).  Section
// 기술 상세 (Technical details): on budget overflow spans are taken in
// descending alpha until the GPU budget holds (here a per-(layer, head) cap,
// ties to the lower span index).
//
// The sigmoid is strictly increasing, so z_S = [alpha_S > tau] is decided as
// a_S > logit(tau) on the score a_S = u . s_S (fp32), with logit(tau) taken in
// fp64 from the fp32 tau, and the budget ranks spans by a_S: the same
// decisions as alpha in exact arithmetic, and still ordered where alpha
// rounds to 1.0f (a_S above ~17).  alpha itself is an optional output.
//
// One workgroup per (b, 512-span chunk, head, layer); each wave scores 64
// spans, one per lane, and writes one mask word with a ballot.  The budget cap
// runs as a second small kernel (route_cap_kernel) on the finished masks.
#include "common.h"

namespace sekv {

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Order-preserving 32-bit key of an fp32 score: unsigned comparison of keys
// is the comparison of the scores (-0 is taken as +0).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// logit(tau) = ln(tau / (1 - tau)) in fp64: alpha > tau exactly when the
// score exceeds it; -inf for tau <= 0, +inf for tau >= 1, NaN for a NaN tau
// (which then routes nothing).
__device__ __forceinline__ double logit_threshold(float tau) {
  if (tau <= 0.f) return -HUGE_VAL;
  if (tau >= 1.f) return HUGE_VAL;
  const double t = (double)tau;
  return log(t) - log1p(-t);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

// Block-wide inclusive scan of one int per thread (256 threads).
__device__ int block_scan256(int v, int* s_tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(v, d);
    if (lane >= d) v += y;
  }
  if (lane == 63) s_tmp[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += s_tmp[w];
  __syncthreads();
  return v + add;
}

// Find the k-th largest key (1-based) among candidates; candidates are given
// by the functor `cand(i, key&)` over i in [0, n).  Returns the key and sets
// k to the rank of the answer among the keys equal to it (1-based).
template <class Cand>
__device__ uint32_t radix_select(int n, int& k, Cand cand, uint32_t* s_hist, int* s_sel) {
  uint32_t prefix = 0, pmask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = threadIdx.x; i < 256; i += 256) s_hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += 256) {
      uint32_t key;
      if (cand(i, key) && (key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int cum = 0, digit = 0;
      for (int bin = 255; bin >= 0; --bin) {
        const int c = (int)s_hist[bin];
        if (cum + c >= k) { digit = bin; break; }
        cum += c;
      }
      s_sel[0] = digit;
      s_sel[1] = k - cum;
    }
    __syncthreads();
    prefix |= (uint32_t)s_sel[0] << shift;
    pmask |= 255u << shift;
    k = s_sel[1];
    __syncthreads();
  }
  return prefix;
}

// The summary keys are streamed once a step: on an index larger than the
// cache holds across steps (NT) their loads carry the non-temporal hint, so
// that they do not evict the cached tables of the kernels that follow (with
// the attention kernel's streamed loads, 775 -> 798 query-tokens/s at 128K).
template <bool NT>
__device__ __forceinline__ float4 load_stream4(const float* p) {
  if constexpr (NT) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 v = __builtin_nontemporal_load((const f32x4*)p);
    return make_float4(v.x, v.y, v.z, v.w);
  } else {
    return *(const float4*)p;
  }
}

// Summary-key dimensions held in registers per lane (d' <= kMaxDp; entries
// past d' are zero, and s_u is zero there, so they add nothing).
constexpr int kMaxDp = 64;

template <int D, int NW, bool NT>
__global__ __launch_bounds__(64 * NW) void route_kernel(const RouteArgs a) {
  __shared__ float s_u[kMaxDp];
  __shared__ double s_thr;
  // workgroup id -> (b, chunk, h) so that every chunk of one (b, h) lands on
  // the same XCD (consecutive ids go round-robin over the 8 XCDs): W^(l,h)
  // and q are then fetched once into that XCD's L2
  const int nchunk = (a.Wd + NW - 1) / NW;
  const int id = blockIdx.x, x8 = id & 7, rest = id >> 3;
  const int chunk = rest % nchunk, bh8 = rest / nchunk;
  const int bh = bh8 * 8 + x8;                 // (b, h) pair, b major
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  if (b >= a.B) return;
  const int lc = blockIdx.y, l = a.layer_begin + lc;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const BMeta bm = a.meta[b];
  const int dp = a.dp;
  const int64_t row = ((int64_t)b * a.layer_count + lc) * a.Hq + h;
  const int wi = chunk * NW + wave;
  const int S = 64 * wi + lane;
  const bool live = wi < a.Wd && S < bm.n_spans;
  // u = W^(l,h) q^(l,h), fp32: NW threads per output, each over D/NW dims.
  // The thread's W row slice and q slice (16-byte loads) are issued first,
  // then the summary keys of this lane's span: u is reduced while the keys
  // are still in flight.
  const float tau_h = a.tau[lc * a.Hq + h];   // first: its logit is taken while the loads below fly
  const float* Wl = a.W + ((int64_t)l * a.Hq + h) * dp * D;
  const bf16_t* qp = a.q + (((int64_t)b * a.layer_count + lc) * a.Hq + h) * D;
  constexpr int QD = D / NW;          // dims per thread
  static_assert(QD >= 8 && QD % 8 == 0, "route: at least 8 dims per thread");
  const int part = threadIdx.x % NW;
  const int j = threadIdx.x / NW;      // dp <= kMaxDp = 64 outputs
  const float* wr = Wl + (int64_t)min(j, dp - 1) * D + part * QD;
  float4 wv[QD / 4];
  uint4 qv[QD / 8];
#pragma unroll
  for (int k = 0; k < QD / 4; ++k) wv[k] = *(const float4*)(wr + 4 * k);
#pragma unroll
  for (int k = 0; k < QD / 8; ++k) qv[k] = *(const uint4*)(qp + part * QD + 8 * k);
  // the lane's span's summary key, 4 dims per 16-byte load (clamped in
  // range; dims past d' meet zeros of u)
  float4 v4[kMaxDp / 4];
  {
    const int d4 = dp_pad4(dp);
    const float* sp = a.s + bm.s_base + ((int64_t)l * a.Hq + h) * d4 * bm.s_pad;
    const int Sc = live ? S : 0;
#pragma unroll
    for (int k = 0; k < kMaxDp / 4; ++k) v4[k] = load_stream4<NT>(sp + skey_index(Sc, 4 * min(k, (d4 >> 2) - 1), d4));
  }
  // logit(tau) once per workgroup, by one lane, while the loads are in flight
  if (threadIdx.x == 0) s_thr = logit_threshold(tau_h);
  __builtin_amdgcn_sched_barrier(0);   // every load issued before the first use
  {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < QD / 4; ++k) {
      const uint32_t q0 = (k & 1) ? qv[k >> 1].z : qv[k >> 1].x;
      const uint32_t q1 = (k & 1) ? qv[k >> 1].w : qv[k >> 1].y;
      acc += wv[k].x * __uint_as_float(q0 << 16) + wv[k].y * __uint_as_float(q0 & 0xffff0000u) +
             wv[k].z * __uint_as_float(q1 << 16) + wv[k].w * __uint_as_float(q1 & 0xffff0000u);
    }
#pragma unroll
    for (int x = 1; x < NW; x <<= 1) acc += __shfl_xor(acc, x);
    if (part == 0) s_u[j] = (j < dp) ? acc : 0.f;   // entries past d' are zero
  }
  __syncthreads();
  if (wi >= a.Wd) return;
  uint64_t* mrow = a.mask + row * a.Wd;
  float* arow = a.alpha ? a.alpha + row * (int64_t)a.Wd * 64 : nullptr;
  float* srow = a.score ? a.score + row * (int64_t)a.Wd * 64 : nullptr;
  const double thr = s_thr;
  float alpha = 0.f, dot = 0.f;
  bool z = false;
  if (live) {
    float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxDp / 4; ++k) {
      d0 += s_u[4 * k] * v4[k].x;
      d1 += s_u[4 * k + 1] * v4[k].y;
      d2 += s_u[4 * k + 2] * v4[k].z;
      d3 += s_u[4 * k + 3] * v4[k].w;
    }
    dot = (d0 + d1) + (d2 + d3);
    z = (double)dot > thr;
    if (arow) alpha = 1.f / (1.f + expf(-dot));
  }
  const uint64_t word = __ballot(z);
  if (lane == 0) mrow[wi] = word;
  if (arow) arow[S] = alpha;
  if (srow) srow[S] = dot;
  // the routed spans' keys, packed per word in span order (the budget
  // kernels then touch only the routed spans)
  if (a.packed && z) a.packed[(row * a.Wd + wi) * 64 + __popcll(word & ((1ull << lane) - 1))] = order_key(dot);
}

// Budget cap, one workgroup per (b, h, lc), after route_kernel: when more than
// cap spans are expanded keep the cap largest scores (the order of alpha),
// ties to the lower span index.  Each candidate is keyed (order key of the
// score, complemented span index): the key order is score descending then
// index ascending, and keys are distinct, so the kept set is exactly the keys
// at or above the cap-th largest key K*.
//  * Collect: thread t takes mask word t and its first 32 packed keys (eight
//    16-byte loads, all issued together; the routing kernel packs the routed
//    spans' keys of each word); a block scan of the per-thread counts places
//    the candidates in LDS in span order.
//  * Select: one histogram of the score keys over the candidates' own range
//    (1024 bins by a shift of (key - min); the keys order like the scores, so
//    the binning is monotone) finds the bin holding K* and how many of its
//    keys are kept; only that bin's keys are then ranked against each other.
//    A boundary bin of more than kCapRank keys (many equal scores) falls back
//    to an 8-pass radix select of the composite keys.
//  * Candidate sets above kCapList fall back to a 4-pass radix select on the
//    score keys over global memory.
constexpr int kCapList = 2048;
constexpr int kCapBins = 1024;
constexpr int kCapRank = 256;

// block_scan256 that also returns the block total.
__device__ int block_scan256_total(int v, int* s_tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(v, d);
    if (lane >= d) v += y;
  }
  if (lane == 63) s_tmp[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += s_tmp[w];
  total = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
  __syncthreads();
  return v + add;
}

// Block-wide inclusive scan of one count per thread (256 threads, counts
// below 2^BITS): wave prefixes by bit-sliced ballots, wave totals through
// s_tmp (4 ints; callers alternate two buffers between consecutive calls, so
// one barrier suffices).
template <int BITS>
__device__ __forceinline__ int block_scan_small(int v, int* s_tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t le = (2ull << lane) - 1;   // lanes <= lane
  int incl = 0, wt = 0;
#pragma unroll
  for (int i = 0; i < BITS; ++i) {
    const uint64_t bal = __ballot((v >> i) & 1);
    incl += (int)__popcll(bal & le) << i;
    wt += (int)__popcll(bal) << i;
  }
  if (lane == 0) s_tmp[wave] = wt;
  __syncthreads();
  int add = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) add += (w < wave) ? s_tmp[w] : 0;
  total = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
  return incl + add;
}

__device__ __forceinline__ float f4_at(const float4& v, int c) {
  return c == 0 ? v.x : (c == 1 ? v.y : (c == 2 ? v.z : v.w));
}

// K* by an 8-pass radix select over the nc composite keys in s_cand (8 bits a
// pass, histograms in LDS).  Returns a threshold T with exactly k keys >= T:
// K* itself, or K*'s leading bytes when the bin of K* is kept whole.
__device__ uint64_t radix_select_keys(const uint64_t* s_cand, int nc, int k, uint32_t* s_hist,
                                      int* s_sel) {
  uint64_t prefix = 0, pmask = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    s_hist[threadIdx.x] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < nc; i0 += 256) {
      // lanes with equal digits are counted with 8 ballots and only the
      // lowest such lane updates the bin (keys share their top bytes, so
      // per-lane atomics would all hit one bin)
      const int i = i0 + threadIdx.x;
      const uint64_t key = (i < nc) ? s_cand[i] : 0ull;
      const bool on = (i < nc) && (key & pmask) == prefix;
      const uint32_t digit = (uint32_t)(key >> shift) & 255u;
      uint64_t peers = __ballot(on);
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const uint64_t bal = __ballot((digit >> bit) & 1u);
        peers &= ((digit >> bit) & 1u) ? bal : ~bal;
      }
      if (on && (peers & ((1ull << lane) - 1)) == 0) atomicAdd(&s_hist[digit], (uint32_t)__popcll(peers));
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns bins 255-4*lane .. 252-4*lane (descending); inclusive scan
      int c[4], tot = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = (int)s_hist[255 - 4 * lane - e];
        tot += c[e];
      }
      int inc = tot;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d);
        if (lane >= d) inc += y;
      }
      const int exc = inc - tot;
      if (exc < k && k <= inc) {   // exactly one lane holds the k-th key
        int cum = exc;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (cum + c[e] >= k) {
            s_sel[0] = 255 - 4 * lane - e;
            s_sel[1] = k - cum;
            s_sel[2] = (k - cum == c[e]);   // every key of the bin is kept
            break;
          }
          cum += c[e];
        }
      }
    }
    __syncthreads();
    prefix |= (uint64_t)s_sel[0] << shift;
    pmask |= 255ull << shift;
    k = s_sel[1];
    const bool whole_bin = s_sel[2] != 0;
    __syncthreads();
    // the cap-th largest key is the smallest of its bin and the whole bin
    // is kept: every key >= prefix (lower bytes zero) is exactly the top cap
    if (whole_bin) break;
  }
  return prefix;
}

__global__ __launch_bounds__(256) void route_cap_kernel(const RouteArgs a) {
  __shared__ uint64_t s_cand[kCapList];
  __shared__ uint32_t s_hist[kCapBins];
  __shared__ unsigned long long s_new[kMaxWords];
  __shared__ uint64_t s_bnd[kCapRank];
  __shared__ uint64_t s_kstar;
  __shared__ uint32_t s_rng[8];
  __shared__ int s_tmp[8];
  __shared__ int s_sel[3];
  __shared__ int s_nb;
  const int b = blockIdx.x, h = blockIdx.y, lc = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const BMeta bm = a.meta[b];
  const int64_t row = ((int64_t)b * a.layer_count + lc) * a.Hq + h;
  uint64_t* mrow = a.mask + row * a.Wd;
  const float* arow = a.score + row * (int64_t)a.Wd * 64;
  for (int w = tid; w < a.Wd; w += 256) s_new[w] = 0ull;
  if (tid == 0) s_nb = 0;
  // collect (mask bits at or past N_S are 0, so their scores are never
  // used): thread t takes mask word t with its first 32 packed keys (the
  // routing kernel packed the routed spans' keys in span order), a block
  // scan of the counts places the candidates in LDS in span order
  const uint4* pk = (const uint4*)(a.packed + row * (int64_t)a.Wd * 64);
  int nc = 0;
  uint32_t lo = 0xffffffffu, hi = 0u;
  int par = 0;
  for (int base = 0; base < a.Wd; base += 256, par ^= 1) {
    const int w = min(base + tid, a.Wd - 1);
    uint64_t bits = mrow[w];
    uint4 kv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kv[i] = pk[w * 16 + i];
    if (base + tid >= a.Wd) bits = 0ull;
    const int c = __popcll(bits);
    int total;
    const int incl = block_scan_small<7>(c, s_tmp + 4 * par, total);
    int pos = nc + incl - c;
    auto put = [&](uint32_t key, int j) {
      if (pos < kCapList) s_cand[pos] = ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)(64 * w + j));
      ++pos;
      lo = min(lo, key);
      hi = max(hi, key);
    };
    // four keys a step; the wave stops once none of its lanes has any left
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (__ballot(bits != 0ull) == 0ull) break;
      const uint32_t vk[4] = {kv[q].x, kv[q].y, kv[q].z, kv[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (bits) {
          const int j = __builtin_ctzll(bits);
          bits &= bits - 1;
          put(vk[e], j);
        }
      }
    }
    // a word with more than 32 routed spans: the rest, four keys a load
    for (int k = 32; bits; k += 4) {
      const uint4 v = pk[w * 16 + (k >> 2)];
      const uint32_t vk[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (bits) {
          const int j = __builtin_ctzll(bits);
          bits &= bits - 1;
          put(vk[e], j);
        }
      }
    }
    nc += total;
  }
  if (nc <= a.cap) return;
  if (nc <= kCapList) {
    // range of the candidates' alpha bits
    lo = __reduce_min_sync(~0ull, lo);
    hi = __reduce_max_sync(~0ull, hi);
    if (lane == 0) {
      s_rng[wave] = lo;
      s_rng[4 + wave] = hi;
    }
    for (int i = tid; i < kCapBins; i += 256) s_hist[i] = 0;
    __syncthreads();
    lo = min(min(s_rng[0], s_rng[1]), min(s_rng[2], s_rng[3]));
    hi = max(max(s_rng[4], s_rng[5]), max(s_rng[6], s_rng[7]));
    const uint32_t range = hi - lo;
    const int sh = max(0, 22 - (int)__clz((int)range));   // (range >> sh) < kCapBins
    auto bin_of = [&](uint64_t key) -> uint32_t { return ((uint32_t)(key >> 32) - lo) >> sh; };
    for (int i = tid; i < nc; i += 256) atomicAdd(&s_hist[bin_of(s_cand[i])], 1u);
    __syncthreads();
    // descending scan: thread t owns bins kCapBins-1-4t .. kCapBins-4-4t
    int cnt[4], tot = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cnt[e] = (int)s_hist[kCapBins - 1 - 4 * tid - e];
      tot += cnt[e];
    }
    int total;
    const int inc = block_scan_small<12>(tot, s_tmp + 4 * par, total);   // tot <= kCapList
    const int exc = inc - tot;
    if (exc < a.cap && a.cap <= inc) {   // exactly one thread holds K*
      int cum = exc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (cum + cnt[e] >= a.cap) {
          s_sel[0] = kCapBins - 1 - 4 * tid - e;
          s_sel[1] = a.cap - cum;   // keys of that bin to keep
          s_sel[2] = cnt[e];
          break;
        }
        cum += cnt[e];
      }
    }
    __syncthreads();
    const uint32_t bstar = (uint32_t)s_sel[0];
    const int r = s_sel[1], m = s_sel[2];
    // keep: bin > bstar, or bin == bstar and key >= kth (kth = 0: whole bin)
    uint64_t kth = 0;
    bool by_bin = true;
    if (r < m) {
      if (m <= kCapRank) {
        for (int i = tid; i < nc; i += 256) {
          const uint64_t key = s_cand[i];
          if (bin_of(key) == bstar) s_bnd[atomicAdd(&s_nb, 1)] = key;
        }
        __syncthreads();
        if (tid < m) {
          const uint64_t e = s_bnd[tid];
          int rank = 0;
          for (int j = 0; j < m; ++j) rank += s_bnd[j] > e;
          if (rank == r - 1) s_kstar = e;
        }
        __syncthreads();
        kth = s_kstar;
      } else {
        kth = radix_select_keys(s_cand, nc, a.cap, s_hist, s_sel);
        by_bin = false;
      }
    }
    for (int i = tid; i < nc; i += 256) {
      const uint64_t key = s_cand[i];
      const uint32_t bk = bin_of(key);
      const bool keep = by_bin ? (bk > bstar || (bk == bstar && key >= kth)) : key >= kth;
      if (keep) {
        const int S = (int)(~(uint32_t)(key & 0xffffffffull));
        atomicOr(&s_new[S >> 6], 1ull << (S & 63));
      }
    }
    __syncthreads();
    for (int w = tid; w < a.Wd; w += 256) mrow[w] = s_new[w];
    return;
  }
  // large candidate sets: radix select on the score keys, ties by span index
  int k = a.cap;
  auto cand = [&](int S, uint32_t& key) -> bool {
    const uint64_t word = mrow[S >> 6];
    if (!((word >> (S & 63)) & 1ull)) return false;
    key = order_key(arow[S]);
    return true;
  };
  const uint32_t vstar = radix_select(bm.n_spans, k, cand, s_hist, s_sel);
  // k = number of spans with key == vstar to keep, lowest span index first
  for (int w = tid; w < a.Wd; w += 256) s_new[w] = mrow[w];
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < a.Wd; base += 256) {
    const int ww = base + tid;
    int tw = 0;
    uint64_t zz = 0;
    if (ww < a.Wd) {
      zz = s_new[ww];
      for (uint64_t bits = zz; bits; bits &= bits - 1)
        tw += (order_key(arow[64 * ww + __builtin_ctzll(bits)]) == vstar);
    }
    int total;
    const int incl = block_scan256_total(tw, s_tmp, total);
    int rank = carry + incl - tw;
    if (ww < a.Wd) {
      uint64_t keep = 0;
      for (uint64_t bits = zz; bits; bits &= bits - 1) {
        const int bit = __builtin_ctzll(bits);
        const uint32_t key = order_key(arow[64 * ww + bit]);
        if (key > vstar) keep |= 1ull << bit;
        else if (key == vstar) {
          if (rank < k) keep |= 1ull << bit;
          ++rank;
        }
      }
      mrow[ww] = keep;
    }
    carry += total;
  }
}

// Budget pooled over a routing call, one 1024-thread workgroup per sequence b,
// after route_kernel: among the routed (layer, head, span) triples of b in the
// call, keep the `budget` largest scores (the order of alpha), ties to the
// lower (layer, head, span) position (the flat order of the mask words).  The budget rule of the
// Technical-details section of the SeKV article, read over the whole call
// instead of one (layer, head).
//  * Collect: the routing kernel has packed the score keys of each word's
//    routed spans at the start of the word's 64 slots, so only routed spans
//    are touched here.  Threads take two mask words a round, each with its
//    first 32 packed keys as eight 16-byte loads, all issued before use;
//    every routed triple (score key, flat position) goes to an LDS list at a
//    slot from one LDS counter per wave (wave prefixes by bit-sliced
//    ballots).  A sequence within its budget stops there.
//  * Radix select of the budget-th largest key over the list, binned over the
//    keys' own range (offsets key - min, at most 11 bits a pass from the top
//    of max - min; the keys order like the scores); once the boundary bin
//    holds at most kPoolRank keys they are ranked against each other instead
//    of binned again.
//  * Keep every larger key.  If the boundary key's equals are not all kept,
//    their positions are ranked against each other and the lowest kept.
// When the routed triples or the halves do not fit in LDS (or the boundary
// has more equal keys than LDS ranks), the passes sweep the mask words and
// scores in global memory in flat order instead: fixed 11, 11, 10-bit passes,
// then a block scan of the equal keys chunk by chunk.
constexpr int kPoolThreads = 1024;
constexpr int kPoolBins = 2048;
constexpr int kPoolList = 12288;    // routed triples held in LDS
constexpr int kPoolHalves = 4096;   // 32-span halves of the new mask held in LDS
constexpr int kPoolRank = 512;      // boundary bins up to this size are ranked directly

// Block-wide inclusive scan over kPoolThreads threads; total = block sum.
__device__ int block_scan_pool(int v, int* s_tmp, int& total) {
  constexpr int NWV = kPoolThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(v, d);
    if (lane >= d) v += y;
  }
  if (lane == 63) s_tmp[wave] = v;
  __syncthreads();
  int add = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const int x = s_tmp[w];
    add += (w < wave) ? x : 0;
    tot += x;
  }
  total = tot;
  __syncthreads();
  return v + add;
}

// Exclusive wave prefix and wave total of per-lane counts below 2^BITS.
template <int BITS>
__device__ __forceinline__ int wave_prefix_pool(int c, int lane, int& total) {
  const uint64_t lt = (1ull << lane) - 1;
  int s = 0, t = 0;
#pragma unroll
  for (int i = 0; i < BITS; ++i) {
    const uint64_t bal = __ballot((c >> i) & 1);
    s += (int)__popcll(bal & lt) << i;
    t += (int)__popcll(bal) << i;
  }
  total = t;
  return s;
}

// The bin of the k-th largest key in s_hist (nbins bins, descending): thread
// i holds bins nbins-1-2i and nbins-2-2i; one thread writes (bin, rank of
// the key within its bin, the bin's count) to s_sel.
__device__ void pool_pick_bin(const uint32_t* s_hist, int nbins, int k, int* s_tmp, int* s_sel) {
  const int hi = nbins - 1 - 2 * (int)threadIdx.x, lo = hi - 1;
  const int chi = (hi >= 0) ? (int)s_hist[hi] : 0;
  const int clo = (lo >= 0) ? (int)s_hist[lo] : 0;
  int tot;
  const int incl = block_scan_pool(chi + clo, s_tmp, tot);
  const int exc = incl - chi - clo;
  if (exc < k && k <= incl) {
    if (exc + chi >= k) {
      s_sel[0] = hi;
      s_sel[1] = k - exc;
      s_sel[2] = chi;
    } else {
      s_sel[0] = lo;
      s_sel[1] = k - exc - chi;
      s_sel[2] = clo;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void load_half(const uint32_t* mh, const float* ab, int64_t t, int64_t nh, uint32_t& bits,
                                          float4 (&av)[8]) {
  const int64_t tc = t < nh ? t : nh - 1;   // in range; a half past the end has no bits
  bits = t < nh ? mh[tc] : 0u;
  const float4* ap = (const float4*)(ab + 32 * tc);
#pragma unroll
  for (int c = 0; c < 8; ++c) av[c] = ap[c];
}

__global__ __launch_bounds__(kPoolThreads) void route_pool_kernel(const RouteArgs a) {
  constexpr int NWV = kPoolThreads / 64;
  __shared__ uint32_t s_hist[kPoolBins];
  __shared__ uint32_t s_key[kPoolList];
  __shared__ int32_t s_pos[kPoolList];
  __shared__ uint32_t s_new[kPoolHalves];
  __shared__ int s_tmp[NWV];
  __shared__ uint32_t s_lo[NWV], s_hi[NWV];
  __shared__ int s_sel[3];
  __shared__ int s_count;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t rows = (int64_t)a.layer_count * a.Hq;
  const int64_t nh = rows * a.Wd * 2;                       // 32-span halves of b's words
  uint32_t* mh = (uint32_t*)(a.mask + (int64_t)b * rows * a.Wd);
  const float* ab = a.score + (int64_t)b * rows * a.Wd * 64;
  int k = a.budget;
  if (tid == 0) s_count = 0;
  for (int i = tid; i < kPoolHalves; i += kPoolThreads) s_new[i] = 0u;
  __syncthreads();
  // ---- collect: thread t takes words t and t + 1024 of a round, each word's
  // first 32 packed keys by eight 16-byte loads (all issued before use), and
  // appends (key, flat position) of its routed spans to the LDS list at a
  // slot from one LDS counter per wave
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  const int64_t nwords = nh >> 1;
  const uint64_t* mw = a.mask + (int64_t)b * rows * a.Wd;
  const uint4* pk = (const uint4*)(a.packed + (int64_t)b * rows * a.Wd * 64);
  auto append = [&](uint64_t bits, const uint4 (&kv)[8], int64_t w, int& pos) {
    // four keys a step; the wave stops once none of its lanes has any left
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (__ballot(bits != 0ull) == 0ull) break;
      const uint32_t vk[4] = {kv[q].x, kv[q].y, kv[q].z, kv[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (bits) {
          const int j = __builtin_ctzll(bits);
          bits &= bits - 1;
          kmin = min(kmin, vk[e]);
          kmax = max(kmax, vk[e]);
          if (pos < kPoolList) {
            s_key[pos] = vk[e];
            s_pos[pos] = (int32_t)(64 * w + j);
          }
          ++pos;
        }
      }
    }
    // a word with more than 32 routed spans: the rest, four keys a load
    for (int k = 32; bits; k += 4) {
      const uint4 v = pk[w * 16 + (k >> 2)];
      const uint32_t vk[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (bits) {
          const int j = __builtin_ctzll(bits);
          bits &= bits - 1;
          kmin = min(kmin, vk[e]);
          kmax = max(kmax, vk[e]);
          if (pos < kPoolList) {
            s_key[pos] = vk[e];
            s_pos[pos] = (int32_t)(64 * w + j);
          }
          ++pos;
        }
      }
    }
  };
  for (int64_t base = 0; base < nwords; base += 2 * kPoolThreads) {
    const int64_t w0 = base + tid, w1 = w0 + kPoolThreads;
    const int64_t c0 = w0 < nwords ? w0 : nwords - 1, c1 = w1 < nwords ? w1 : nwords - 1;   // in range
    uint64_t bits0 = mw[c0], bits1 = mw[c1];
    uint4 kv0[8], kv1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kv0[i] = pk[c0 * 16 + i];
      kv1[i] = pk[c1 * 16 + i];
    }
    if (w0 >= nwords) bits0 = 0ull;
    if (w1 >= nwords) bits1 = 0ull;
    int wt;
    const int pre = wave_prefix_pool<8>(__popcll(bits0) + __popcll(bits1), lane, wt);
    int wb = 0;
    if (lane == 0 && wt > 0) wb = atomicAdd(&s_count, wt);
    int pos = __shfl(wb, 0) + pre;
    append(bits0, kv0, w0, pos);
    append(bits1, kv1, w1, pos);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, d));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d));
  }
  if (lane == 0) {
    s_lo[wave] = kmin;
    s_hi[wave] = kmax;
  }
  __syncthreads();
  const int total = s_count;
  if (total <= k) return;   // uniform: b is within its budget
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    kmin = min(kmin, s_lo[w]);
    kmax = max(kmax, s_hi[w]);
  }
  uint32_t vstar = 0u;
  if (total <= kPoolList && nh <= kPoolHalves) {
    // ---- radix select over the LDS list, binned over [kmin, kmax]
    const uint32_t r = kmax - kmin;
    const int nb = r ? 32 - __clz((int)r) : 0;
    uint32_t prefix = 0, pmask = 0;
    int ceq = total;   // keys equal to the selected one
    bool ranked = false;
    for (int top = nb; top > 0; top -= 11) {
      const int shift = max(top - 11, 0), nbins = 1 << (top - shift);
      for (int i = tid; i < kPoolBins; i += kPoolThreads) s_hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < total; i += kPoolThreads) {
        const uint32_t o = s_key[i] - kmin;
        if ((o & pmask) == prefix) atomicAdd(&s_hist[(o >> shift) & (uint32_t)(nbins - 1)], 1u);
      }
      __syncthreads();
      pool_pick_bin(s_hist, nbins, k, s_tmp, s_sel);
      prefix |= (uint32_t)s_sel[0] << shift;
      pmask |= (uint32_t)(nbins - 1) << shift;
      k = s_sel[1];
      ceq = s_sel[2];
      __syncthreads();
      if (shift > 0 && ceq <= kPoolRank) {   // uniform
        // a small boundary bin: its keys ranked against each other give the
        // boundary key, its rank among equals and their count at once
        if (tid == 0) s_count = 0;
        __syncthreads();
        for (int i = tid; i < total; i += kPoolThreads) {
          const uint32_t o = s_key[i] - kmin;
          if ((o & pmask) == prefix) s_hist[atomicAdd(&s_count, 1)] = s_key[i];
        }
        __syncthreads();
        for (int i = tid; i < ceq; i += kPoolThreads) {
          const uint32_t ki = s_hist[i];
          int gt = 0, ge = 0;
          for (int j = 0; j < ceq; ++j) {
            const uint32_t kj = s_hist[j];
            gt += kj > ki;
            ge += kj >= ki;
          }
          if (gt < k && k <= ge) {   // every thread holding this key writes the same
            s_sel[0] = (int)ki;
            s_sel[1] = k - gt;
            s_sel[2] = ge - gt;
          }
        }
        __syncthreads();
        ranked = true;
        vstar = (uint32_t)s_sel[0];
        k = s_sel[1];
        ceq = s_sel[2];
        __syncthreads();
        break;
      }
    }
    if (!ranked) vstar = kmin + prefix;
    // ---- keep: every larger key, and the k lowest-position equal keys
    bool done = false;
    if (k == ceq) {
      for (int i = tid; i < total; i += kPoolThreads)
        if (s_key[i] >= vstar) {
          const int p = s_pos[i];
          atomicOr(&s_new[p >> 5], 1u << (p & 31));
        }
      done = true;
    } else if (ceq <= kPoolBins) {
      // the equal keys' positions (in s_hist), each ranked against the others
      if (tid == 0) s_count = 0;
      __syncthreads();
      for (int i = tid; i < total; i += kPoolThreads) {
        const uint32_t key = s_key[i];
        const int p = s_pos[i];
        if (key > vstar) atomicOr(&s_new[p >> 5], 1u << (p & 31));
        else if (key == vstar) s_hist[atomicAdd(&s_count, 1)] = (uint32_t)p;
      }
      __syncthreads();
      for (int e = tid; e < ceq; e += kPoolThreads) {
        const uint32_t p = s_hist[e];
        int rank = 0;
        for (int f = 0; f < ceq; ++f) rank += s_hist[f] < p;
        if (rank < k) atomicOr(&s_new[p >> 5], 1u << (p & 31));
      }
      done = true;
    }
    if (done) {   // uniform
      __syncthreads();
      for (int i = tid; i < (int)nh; i += kPoolThreads) mh[i] = s_new[i];
      return;
    }
  } else {
    // ---- radix select sweeping global memory: fixed 11, 11, 10-bit digits
    uint32_t prefix = 0, pmask = 0;
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int nbins = pass == 2 ? 1024 : 2048;
      for (int i = tid; i < kPoolBins; i += kPoolThreads) s_hist[i] = 0;
      __syncthreads();
      for (int64_t t = tid; t < nh; t += kPoolThreads) {
        uint32_t bits;
        float4 av[8];
        load_half(mh, ab, t, nh, bits, av);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const uint32_t key = order_key(f4_at(av[j >> 2], j & 3));
          if (((bits >> j) & 1u) && (key & pmask) == prefix)
            atomicAdd(&s_hist[(key >> shift) & (uint32_t)(nbins - 1)], 1u);
        }
      }
      __syncthreads();
      pool_pick_bin(s_hist, nbins, k, s_tmp, s_sel);
      prefix |= (uint32_t)s_sel[0] << shift;
      pmask |= (uint32_t)(nbins - 1) << shift;
      k = s_sel[1];
      __syncthreads();
    }
    vstar = prefix;
  }
  // ---- keep, sweeping global memory in flat order: every larger key, and
  // the k lowest-position keys equal to vstar (block scan of their counts)
  int carry = 0;
  for (int64_t base = 0; base < nh; base += kPoolThreads) {
    const int64_t t = base + tid;
    uint32_t bits, keep = 0u, eq = 0u;
    float4 av[8];
    load_half(mh, ab, t, nh, bits, av);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t key = order_key(f4_at(av[j >> 2], j & 3));
      const bool on = (bits >> j) & 1u;
      keep |= (uint32_t)(on && key > vstar) << j;
      eq |= (uint32_t)(on && key == vstar) << j;
    }
    const int ne = __popc(eq);
    int chunk;
    int rank = carry + block_scan_pool(ne, s_tmp, chunk) - ne;
    for (uint32_t x = eq; x; x &= x - 1) {
      if (rank < k) keep |= 1u << __builtin_ctz(x);
      ++rank;
    }
    if (t < nh && bits != 0u) mh[t] = keep;
    carry += chunk;
  }
}

// tau^(l,h): midpoint of the k-th and (k+1)-th largest alpha over every
// (b, span), k = round(frac * N) clipped to [1, N - 1].
__global__ __launch_bounds__(256) void calibrate_kernel(const CalibArgs a) {
  __shared__ uint32_t s_hist[256];
  __shared__ int s_sel[2];
  const int h = blockIdx.x, lc = blockIdx.y;
  int64_t N = 0;
  for (int b = 0; b < a.B; ++b) N += a.meta[b].n_spans;
  int k = (int)floor((double)a.frac * (double)N + 0.5);
  k = max(1, min(k, (int)N - 1));
  // flatten (b, S) into one index range via a per-b walk
  auto cand = [&](int i, uint32_t& key) -> bool {
    int b = 0, rem = i;
    while (b < a.B && rem >= a.meta[b].n_spans) { rem -= a.meta[b].n_spans; ++b; }
    if (b >= a.B) return false;
    key = __float_as_uint(a.alpha[(((int64_t)b * a.layer_count + lc) * a.Hq + h) * (int64_t)a.Wd * 64 + rem]);
    return true;
  };
  int k1 = k, k2 = k + 1;
  const uint32_t v1 = radix_select((int)N, k1, cand, s_hist, s_sel);
  const uint32_t v2 = radix_select((int)N, k2, cand, s_hist, s_sel);
  if (threadIdx.x == 0)
    a.tau_out[lc * a.Hq + h] = 0.5f * (__uint_as_float(v1) + __uint_as_float(v2));
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  // 8 waves (mask words) per workgroup: at 128K tokens the 32 heads of a
  // layer take 192 workgroups, one per CU, and W^(l,h) is read by 6
  // workgroups per head instead of 11 (measured 0.9 us faster per launch
  // than 4 waves; 2 and 16 were slower)
  constexpr int NW = 8;
  const int nchunk = (a.Wd + NW - 1) / NW;
  const int nbh8 = (a.B * a.Hq + 7) / 8;
  const dim3 grid(nbh8 * 8 * nchunk, a.layer_count);
  if (a.D == 128 && a.stream) hipLaunchKernelGGL((route_kernel<128, NW, true>), grid, dim3(64 * NW), 0, st, a);
  else if (a.D == 128) hipLaunchKernelGGL((route_kernel<128, NW, false>), grid, dim3(64 * NW), 0, st, a);
  else if (a.D == 64 && a.stream) hipLaunchKernelGGL((route_kernel<64, NW, true>), grid, dim3(64 * NW), 0, st, a);
  else if (a.D == 64) hipLaunchKernelGGL((route_kernel<64, NW, false>), grid, dim3(64 * NW), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_route_cap(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(route_cap_kernel, dim3(a.B, a.Hq, a.layer_count), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_route_pool(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(route_pool_kernel, dim3(a.B), dim3(kPoolThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_calibrate(const CalibArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(calibrate_kernel, dim3(a.Hq, a.layer_count), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sekv
