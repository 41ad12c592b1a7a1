// Randomized truncated SVD of the span matrices, gfx950.
//
// SeKV article (aitrends.kr/articles/75020), section 방법론 (Method): every
// span's key and value matrix gets a truncated SVD per layer and head, and
// the SVD is randomized so that the prefill cost parallelises.  Section
// 기술 상세 (Technical details): Khat_S = sum_i m_i sigma_i u_i v_i^T, so
// sigma_i * m_i is stored beside the factors.
//
// Method: randomized subspace iteration (Halko, Martinsson and Tropp,
// "Finding structure with randomness", SIAM Review 2011) on the right
// singular subspace of one span matrix A (n x d, bf16).  With sketch width
// l = min(R + p, n, d):
//   Z = Omega (d x l, N(0, 1));  q + 1 times: Z <- orth(A^T (A Z));
//   C = A Z;  C^T C = E Lambda E^T (Rayleigh-Ritz, cyclic Jacobi);
//   V = Z E (first R columns by decreasing eigenvalue), sigma = sqrt(lambda),
//   U = orth(A V Sigma^-1) (Cholesky-QR).
// When l = min(n, d) the sketch already spans A's row space: Z = orth(A^T)
// for n <= d, Z = I for n > d.
//
// The products with A are the dense contractions and run on MFMA: A is
// staged 32 rows at a time in LDS, row-major for A Z (16x16x32 bf16, A as the
// A operand) and transposed for A^T Y (16x16x16 bf16).  A is exact in bf16;
// the fp32 right-hand operands are split into bf16 terms (x = t0 + t1 [+ t2],
// each term the rounding of the remainder): two terms (16 mantissa bits) in
// the range finder, three (fp32 accuracy) for the Rayleigh-Ritz and U.
// Orthonormalisation is Cholesky-QR with an fp64 Gram matrix and fp64
// factorisation (columns whose pivot falls below 1e-14 of the largest are
// dropped as numerically dependent); one pass per step keeps the basis
// orthonormal to ~5e-6 at these sketch widths (the exact-range case, whose
// Gram is that of A itself, gets a second pass).  Grams of C and U
// accumulate fp32 products in fp64.
//
// Omega ~ N(0, 1) from Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011) keyed by the seed
// and counter (matrix id, element), through the Box-Muller transform.
//
// One workgroup (256 threads) per matrix.
#include "common.h"

namespace sekv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_k32(u32x4_t a, u32x4_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(u32x2_t a, u32x2_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a),
                                                   __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bfv(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ uint32_t rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ bf16_t to_bf(float x) { return (bf16_t)rne(x); }

// x = t[0] + t[1] + ... + remainder, each term the bf16 rounding of what is left.
template <int NT>
__device__ __forceinline__ void split_terms(float x, uint32_t (&t)[NT]) {
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    t[i] = rne(x);
    x -= bfv(t[i]);
  }
}

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

// Lower-triangle index e -> (r, c) with c <= r.
__device__ __forceinline__ void tri_decode(int e, int& r, int& c) {
  r = (int)((sqrtf(8.f * (float)e + 1.f) - 1.f) * 0.5f);
  while (r * (r + 1) / 2 > e) --r;
  while ((r + 1) * (r + 2) / 2 <= e) ++r;
  c = e - r * (r + 1) / 2;
}

// Rows of A staged per chunk: 32, or 16 when the sketch is at most 32 wide
// (the smaller staging area then lets four workgroups share a CU instead of
// three; for wider sketches 16 rows save too little LDS to add one).
template <int LP>
struct Chunk {
  static constexpr int NC = LP <= 48 ? 16 : 32;
  static constexpr int NRT = NC / 16;   // 16-row tiles per chunk
};

// LDS layout (bytes).
//   ZT  float [LP][D + 4]   basis columns as rows (Z^T), later V^T
//   X   Ar  bf16 [kNC][D + 8]  staged rows of A (row-major, A operand)
//       then At bf16 [D/16][kNRT][64][4] (A^T operand) + Yb hi/lo
//            bf16 [kNRT][LP/16][64][4] each (range finder),
//       or CT float [LP][kNC + 4] (a chunk of A Z or of U'),
//       or Lf float [LP][LP] (Cholesky factor transposed, fp32, during orth)
//   G   double [JP][JP]  Gram / Cholesky factor (lower), L^-1 (upper);
//       or T float [JP][JP + 1] (Jacobi), with E^T float [JP][EP] in X when
//       it fits there (X is idle during the Jacobi), else after T;
//       finally Lt float [LP][LP] (L^-T for U, at least this many bytes).
//   JP = the largest sketch width min(R + p, d) rounded up to even, so the
//   small-matrix region is sized by the sketch, not by its 16-wide padding
//   (at R = 32, p = 8: 40 instead of 48; this region decides how many
//   workgroups share a CU).
template <int D, int LP>
struct Lay {
  static constexpr int kNC = Chunk<LP>::NC;
  static constexpr int ZP = D + 4;
  static constexpr int ARP = D + 8;
  static constexpr int CTP = kNC + 4;
  static constexpr size_t zt = 0;
  static constexpr size_t x = zt + (size_t)LP * ZP * 4;
  static constexpr size_t at = x + (size_t)kNC * ARP * 2;
  static constexpr size_t yb = at + (size_t)kNC * D * 2;
  static constexpr size_t yb_terms = (size_t)kNC * LP;   // bf16 elements per term
  static constexpr size_t ct = at;
  static constexpr size_t x_end1 = yb + 2 * yb_terms * 2;
  static constexpr size_t x_end2 = ct + (size_t)LP * CTP * 4;
  static constexpr size_t x_end3 = x + (size_t)LP * LP * 4;
  static constexpr size_t x_end = ((x_end1 > x_end2 ? x_end1 : x_end2) > x_end3
                                       ? (x_end1 > x_end2 ? x_end1 : x_end2) : x_end3);
  static constexpr size_t g = (x_end + 15) & ~(size_t)15;
};

// The runtime part of the layout: pitches of the small matrices for sketch
// widths up to lmax (<= LP), where E^T goes, and the workgroup's LDS bytes.
struct SmallLay {
  int jp, tp, ep;      // G pitch and Jacobi size (even), T pitch, E^T pitch
  size_t et;           // byte offset of E^T, followed by the Jacobi's rotation
                       // list (jp / 2 + 1 f32x4)
  size_t bytes;        // dynamic LDS of the workgroup
};
template <int D, int LP>
__host__ __device__ inline SmallLay small_lay(int lmax) {
  using Y = Lay<D, LP>;
  SmallLay r;
  r.jp = lmax + (lmax & 1);
  r.tp = r.jp + 1;
  r.ep = ((r.jp + 3) & ~3) + 4;
  const int np = r.jp / 2;
  const size_t gb = (size_t)r.jp * r.jp * 8, tb = (size_t)r.jp * r.tp * 4;
  const size_t eb = (size_t)r.jp * r.ep * 4 + (size_t)(np + 1) * 16;
  if (eb <= Y::g - Y::x) {
    r.et = Y::x;
    r.bytes = Y::g + (gb > tb ? gb : tb);
  } else {
    r.et = Y::g + ((tb + 15) & ~(size_t)15);
    r.bytes = r.et + eb > Y::g + gb ? r.et + eb : Y::g + gb;
  }
  // the fp32 L^-T table of the U step, [LP][LP] over the G region
  const size_t lt = (size_t)LP * LP * 4;
  if (r.bytes < Y::g + lt) r.bytes = Y::g + lt;
  return r;
}

// Stage rows [c0, c0 + kNC) of A (rows >= n read as zero) into Ar and, for
// the range finder, into the transposed operand tiles At.
template <int D, int kNC, bool WITH_AT>
__device__ void stage(const bf16_t* __restrict__ A, int n, int c0, bf16_t* Ar, bf16_t* At) {
  constexpr int kNRT = kNC / 16;
  constexpr int CPR = D / 8;
  constexpr int ARP = D + 8;
  for (int u = threadIdx.x; u < kNC * CPR; u += 256) {
    const int r = u / CPR, c8 = (u - r * CPR) * 8;
    const int row = c0 + r;
    u32x4_t v = *(const u32x4_t*)(A + (int64_t)min(row, n - 1) * D + c8);
    if (row >= n) v = u32x4_t{0u, 0u, 0u, 0u};
    *(u32x4_t*)(Ar + r * ARP + c8) = v;
    if (WITH_AT) {
      const int base = (r >> 4) * 64 * 4 + 16 * ((r & 15) >> 2) * 4 + (r & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dim = c8 + e;
        const uint32_t h = (e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xffffu);
        At[(dim >> 4) * (kNRT * 64 * 4) + base + (dim & 15) * 4] = (bf16_t)h;
      }
    }
  }
}

// B operand of 16x16x32 for columns [16 jt, 16 jt + 16) and dims
// [32 ks, 32 ks + 32) of Z, read from the rows of ZT, in NT bf16 terms.
template <int D, int NT>
__device__ __forceinline__ void z_operand(const float* ZT, int jt, int ks, int lane, u32x4_t (&o)[NT]) {
  const float* p = ZT + (jt * 16 + (lane & 15)) * (D + 4) + ks * 32 + 8 * (lane >> 4);
  const f32x4 v0 = *(const f32x4*)p, v1 = *(const f32x4*)(p + 4);
  const float x[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  uint32_t t[8][NT];
#pragma unroll
  for (int e = 0; e < 8; ++e) split_terms<NT>(x[e], t[e]);
#pragma unroll
  for (int k = 0; k < NT; ++k)
    o[k] = u32x4_t{t[0][k] | (t[1][k] << 16), t[2][k] | (t[3][k] << 16), t[4][k] | (t[5][k] << 16),
                   t[6][k] | (t[7][k] << 16)};
}

// One 16 x 16 tile of (A_chunk Z): rows [16 rt, 16 rt + 16) of the staged
// chunk, columns [16 jt, 16 jt + 16); D layout (lane = col + 16 (row / 4)).
template <int D, int NT>
__device__ __forceinline__ f32x4 az_tile(const bf16_t* Ar, const float* ZT, int rt, int jt, int lane) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const u32x4_t av = *(const u32x4_t*)(Ar + (rt * 16 + (lane & 15)) * (D + 8) + ks * 32 + 8 * (lane >> 4));
    u32x4_t zb[NT];
    z_operand<D, NT>(ZT, jt, ks, lane, zb);
#pragma unroll
    for (int k = 0; k < NT; ++k) acc = mfma_k32(av, zb[k], acc);
  }
  return acc;
}

// ZT <- rows of A^T (A Z) (all columns of Z; unused columns of Z are zero).
template <int D, int LP>
__device__ __forceinline__ void range_step_body(const bf16_t* __restrict__ A, int n, uint8_t* lds) {
  constexpr int kNC = Chunk<LP>::NC, kNRT = Chunk<LP>::NRT;
  using Y = Lay<D, LP>;
  constexpr int NJT = LP / 16, NDT = D / 16, DTW = (NDT + 3) / 4;
  float* ZT = (float*)(lds + Y::zt);
  bf16_t* Ar = (bf16_t*)(lds + Y::x);
  bf16_t* At = (bf16_t*)(lds + Y::at);
  bf16_t* Yh = (bf16_t*)(lds + Y::yb);
  bf16_t* Yl = Yh + Y::yb_terms;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  f32x4 w[DTW][NJT];
#pragma unroll
  for (int i = 0; i < DTW; ++i)
#pragma unroll
    for (int j = 0; j < NJT; ++j) w[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < n; c0 += kNC) {
    stage<D, kNC, true>(A, n, c0, Ar, At);
    __syncthreads();
    for (int t = wave; t < kNRT * NJT; t += 4) {
      const int rt = t / NJT, jt = t - rt * NJT;
      const f32x4 y = az_tile<D, 2>(Ar, ZT, rt, jt, lane);
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = rne(y[e]);
        l[e] = rne(y[e] - bfv(h[e]));
      }
      const int o = ((rt * NJT + jt) * 64 + lane) * 4;
      *(u32x2_t*)(Yh + o) = u32x2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      *(u32x2_t*)(Yl + o) = u32x2_t{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
    }
    __syncthreads();
#pragma unroll
    for (int di = 0; di < DTW; ++di) {
      const int dt = wave + 4 * di;
      if (dt < NDT) {
#pragma unroll
        for (int rt = 0; rt < kNRT; ++rt) {
          const u32x2_t av = *(const u32x2_t*)(At + ((dt * kNRT + rt) * 64 + lane) * 4);
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt) {
            const int o = ((rt * NJT + jt) * 64 + lane) * 4;
            w[di][jt] = mfma_k16(av, *(const u32x2_t*)(Yh + o), w[di][jt]);
            w[di][jt] = mfma_k16(av, *(const u32x2_t*)(Yl + o), w[di][jt]);
          }
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int di = 0; di < DTW; ++di) {
    const int dt = wave + 4 * di;
    if (dt < NDT) {
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
        *(f32x4*)(ZT + (jt * 16 + (lane & 15)) * Y::ZP + dt * 16 + 4 * (lane >> 4)) = w[di][jt];
    }
  }
  __syncthreads();
}

template <int D, int LP>
__device__ __noinline__ void range_step_call(const bf16_t* __restrict__ A, int n, uint8_t* lds) {
  range_step_body<D, LP>(A, n, lds);
}
template <int D, int LP>
__device__ __forceinline__ void range_step(const bf16_t* __restrict__ A, int n, uint8_t* lds) {
  if constexpr (LP >= 48) range_step_body<D, LP>(A, n, lds);
  else range_step_call<D, LP>(A, n, lds);
}

// In-place Cholesky (LDL^T form) of the leading m x m block of the symmetric
// fp64 matrix G (pitch GP; both triangles filled on entry; the lower
// triangle is updated).  Afterwards L_jk = G[j][k] * dinv[k] (j > k), L_kk =
// 1 / dinv[k]; a pivot at or below 1e-14 of the largest diagonal marks a
// dependent column: dinv = 0 there.
//
// Right-looking, two columns per barrier: step (k, k + 1) applies both
// rank-one updates to the trailing block (rows and columns >= k + 2) at once,
// forming column k + 1 after the first update on the fly from the old
// values; that column is written back during the next step (nothing reads it
// there), so the columns being read are never written within a step.
__device__ void cholesky64(double* G, int m, int GP, float* dinv) {
  // largest diagonal: each wave reads it in parallel and reduces by shuffles
  double maxd = 0.0;
  for (int i = threadIdx.x & 63; i < m; i += 64) maxd = fmax(maxd, G[i * GP + i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) maxd = fmax(maxd, __shfl_xor(maxd, o));
  const double tol = 1e-14 * maxd;
  const int tid = threadIdx.x;
  __syncthreads();
  auto pivot_inv = [&](double d) { return (d > tol && d > 0.0) ? 1.0 / d : 0.0; };
  // write back column c (the second of step (c - 1, c)) after its update by
  // column c - 1, whose pivot inverse inv0 the previous step formed
  auto write_back = [&](int c, double inv0) {
    const double a = G[c * GP + c - 1];
    for (int i = c + tid; i < m; i += 256)
      G[i * GP + c] -= G[i * GP + c - 1] * a * inv0;   // i == c: the diagonal, a * a * inv0
  };
  double inv_prev = 0.0;   // pivot inverse of the first column of the previous step
  for (int k = 0; k < m; k += 2) {
    if (k >= 2) write_back(k - 1, inv_prev);
    if (k + 1 < m) {
      const double inv0 = pivot_inv(G[k * GP + k]);
      inv_prev = inv0;
      const double a = G[(k + 1) * GP + k];
      const double inv1 = pivot_inv(G[(k + 1) * GP + k + 1] - a * a * inv0);
      for (int i = k + 2 + (tid >> 2); i < m; i += 64) {
        const double ci0 = G[i * GP + k];
        const double ci1 = G[i * GP + k + 1] - ci0 * a * inv0;
        const double f0 = ci0 * inv0, f1 = ci1 * inv1;
        for (int j = k + 2 + (tid & 3); j <= i; j += 4) {
          const double cj0 = G[j * GP + k];
          const double cj1 = G[j * GP + k + 1] - cj0 * a * inv0;
          G[i * GP + j] -= f0 * cj0 + f1 * cj1;
        }
      }
    }
    __syncthreads();
  }
  if (m >= 2 && (m & 1) == 0) {   // the last step's second column
    write_back(m - 1, inv_prev);
    __syncthreads();
  }
  for (int k = tid; k < m; k += 256) {
    const double dk = G[k * GP + k];
    dinv[k] = (dk > tol && dk > 0.0) ? (float)(1.0 / sqrt(dk)) : 0.f;
  }
  __syncthreads();
}

// Orthonormalise the first m rows of ZT (columns of Z, length D) in place:
// Cholesky-QR, Z <- Z L^-T.  Rows m..LP-1 of ZT are zero on entry and exit.
template <int D, int LP>
__device__ __forceinline__ void orthonormalize_body(uint8_t* lds, int m, int GP, float* dinv) {
  using Y = Lay<D, LP>;
  float* ZT = (float*)(lds + Y::zt);
  double* G = (double*)(lds + Y::g);
  float* Lf = (float*)(lds + Y::x);
  const int nb = (m + 1) >> 1, nblk = nb * (nb + 1) / 2;
  for (int t = threadIdx.x; t < nblk; t += 256) {
    int bj, bi;
    tri_decode(t, bj, bi);
    const float* r0 = ZT + 2 * bi * Y::ZP;
    const float* r1 = r0 + Y::ZP;
    const float* q0 = ZT + 2 * bj * Y::ZP;
    const float* q1 = q0 + Y::ZP;
    double g00 = 0.0, g01 = 0.0, g10 = 0.0, g11 = 0.0;
    for (int d = 0; d < D; d += 4) {
      const f32x4 a0 = *(const f32x4*)(r0 + d), a1 = *(const f32x4*)(r1 + d);
      const f32x4 b0 = *(const f32x4*)(q0 + d), b1 = *(const f32x4*)(q1 + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g00 += (double)a0[e] * (double)b0[e];
        g01 += (double)a0[e] * (double)b1[e];
        g10 += (double)a1[e] * (double)b0[e];
        g11 += (double)a1[e] * (double)b1[e];
      }
    }
    const int i0 = 2 * bi, j0 = 2 * bj;
    G[i0 * GP + j0] = g00; G[j0 * GP + i0] = g00;
    G[i0 * GP + j0 + 1] = g01; G[(j0 + 1) * GP + i0] = g01;
    G[(i0 + 1) * GP + j0] = g10; G[j0 * GP + i0 + 1] = g10;
    G[(i0 + 1) * GP + j0 + 1] = g11; G[(j0 + 1) * GP + i0 + 1] = g11;
  }
  __syncthreads();
  cholesky64(G, m, GP, dinv);
  // Lf[j][k] = L[k][j] (j < k < m): row j holds the multipliers of column j
  for (int e = threadIdx.x; e < LP * LP; e += 256) {
    const int j = e / LP, k = e - j * LP;
    Lf[e] = (j < k && k < m) ? (float)G[k * GP + j] * dinv[j] : 0.f;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    float w[LP];
#pragma unroll
    for (int j = 0; j < LP; ++j) w[j] = ZT[j * Y::ZP + d];
#pragma unroll
    for (int j = 0; j < LP; ++j) {
      if (j < m) {
        const float zj = w[j] * dinv[j];
        w[j] = zj;
#pragma unroll
        for (int k = j + 1; k < LP; ++k) w[k] -= Lf[j * LP + k] * zj;
      } else {
        w[j] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < LP; ++j) ZT[j * Y::ZP + d] = w[j];
  }
  __syncthreads();
}

template <int D, int LP>
__device__ __noinline__ void orthonormalize_call(uint8_t* lds, int m, int GP, float* dinv) {
  orthonormalize_body<D, LP>(lds, m, GP, dinv);
}
// Inlined into the kernel for sketches of 48 columns and more (measured 18.4
// -> 18.0 ms per 128K layer at R = 32, and fewer registers than the call
// needs); a call for narrower ones, whose kernels would otherwise grow past
// the 128 registers that four workgroups per CU allow.
template <int D, int LP>
__device__ __forceinline__ void orthonormalize(uint8_t* lds, int m, int GP, float* dinv) {
  if constexpr (LP >= 48) orthonormalize_body<D, LP>(lds, m, GP, dinv);
  else orthonormalize_call<D, LP>(lds, m, GP, dinv);
}

// Cyclic Jacobi eigen-decomposition of the symmetric l x l matrix T (pitch
// TP; rows and columns l..JP-1 zero, JP even >= l).  Eigenvectors are
// accumulated as the rows of ET (pitch EP): row p of ET is column p of E.  The disjoint
// pairs of a round (round-robin ordering) rotate together; each 2 x 2 block
// of T and each 4-element piece of a pair of ET rows is one work item.
template <int LP>
__device__ void jacobi(float* T, float* ET, int l, int JP, int TP, int EP, f32x4* rot, int* rflag) {
  constexpr int NPM = LP / 2;                                 // pairs at most
  constexpr int TT = (NPM * (NPM + 1) / 2 + 255) / 256;       // T blocks per thread
  constexpr int TE = (NPM * ((LP + 3) / 4) + 255) / 256;      // E^T pieces per thread
  const int m = l + (l & 1);
  const int np = m >> 1;
  const int nrc = (l + 3) >> 2;
  const int nblk = np * (np + 1) / 2;   // pairs of pairs k1 <= k2
  for (int i = threadIdx.x; i < JP * EP; i += 256) ET[i] = (i / EP == i % EP) ? 1.f : 0.f;
  // this thread's tasks, the same every round: T blocks t = tid + 256 u
  // (k1 | k2 << 8) and E^T pieces (pair k | first row r0 << 8); -1 for none
  int tk[TT], te[TE];
#pragma unroll
  for (int u = 0; u < TT; ++u) {
    const int t = threadIdx.x + 256 * u;
    int k2 = 0, k1 = 0;
    if (t < nblk) tri_decode(t, k2, k1);
    tk[u] = (t < nblk) ? (k1 | (k2 << 8)) : -1;
  }
#pragma unroll
  for (int u = 0; u < TE; ++u) {
    const int t = threadIdx.x + 256 * u, k = t / max(nrc, 1);
    te[u] = (t < np * nrc) ? (k | ((4 * (t - k * nrc)) << 8)) : -1;
  }
  // rflag[r & 1]: a pair of round r rotates (a round without rotation skips
  // its updates); the other slot is cleared during the round for the next
  if (threadIdx.x < 2) rflag[threadIdx.x] = 0;
  __syncthreads();
  int r_all = 0;
  for (int sweep = 0; sweep < 12; ++sweep) {
    // a sweep rotates iff some pair meets the rotation test on the sweep's
    // starting T (a round without rotation leaves T as it was): after the
    // first sweep, one pass over the pairs decides it instead of a sweep of
    // rounds that all skip
    if (sweep > 0) {
      int need = 0;
      for (int e = threadIdx.x; e < l * l; e += 256) {
        const int p = e / l, q = e - p * l;
        if (p < q) {
          const float apq = T[p * TP + q], app = T[p * TP + p], aqq = T[q * TP + q];
          need |= (apq * apq > 1e-14f * fabsf(app * aqq) && fabsf(apq) > 1e-30f);
        }
      }
      if (!__syncthreads_or(need)) break;
    }
    for (int rnd = 0; rnd + 1 < m; ++rnd, ++r_all) {
      if (threadIdx.x < np) {
        const int k = threadIdx.x;
        int pp = k - 1 + rnd;
        if (pp >= m - 1) pp -= m - 1;
        int qq = m - 2 - k + rnd;
        if (qq >= m - 1) qq -= m - 1;
        const int p = (k == 0) ? 0 : pp + 1, q = qq + 1;
        float c = 1.f, s = 0.f;
        if (p < l && q < l) {
          const float apq = T[p * TP + q], app = T[p * TP + p], aqq = T[q * TP + q];
          // rotate when |apq| > 1e-7 sqrt|app aqq| (squared: no root); the
          // angle from hardware reciprocal and root, since c and s are then
          // formed from t as an exact rotation (c^2 + s^2 = 1 to rounding)
          if (apq * apq > 1e-14f * fabsf(app * aqq) && fabsf(apq) > 1e-30f) {
            const float th = (aqq - app) * __builtin_amdgcn_rcpf(2.f * apq);
            const float t = (th >= 0.f ? 1.f : -1.f) *
                            __builtin_amdgcn_rcpf(fabsf(th) + __builtin_amdgcn_sqrtf(1.f + th * th));
            c = rsqrtf(1.f + t * t);
            s = t * c;
            rflag[r_all & 1] = 1;
          }
        }
        rot[k] = f32x4{c, s, __int_as_float(p), __int_as_float(q)};
      }
      __syncthreads();
      // the round flag and the rotations of this thread's tasks, read together
      const bool rotates = rflag[r_all & 1] != 0;
      f32x4 ra[TT], rb[TT], rc[TE];
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const int kk = tk[u] < 0 ? 0 : tk[u];
        ra[u] = rot[kk & 255];
        rb[u] = rot[kk >> 8];
      }
#pragma unroll
      for (int u = 0; u < TE; ++u) rc[u] = rot[(te[u] < 0 ? 0 : te[u]) & 255];
      if (threadIdx.x == 0) rflag[(r_all + 1) & 1] = 0;
      if (!rotates) {
        __syncthreads();
        continue;
      }
      // T is symmetric: each pair of pairs k1 <= k2 updates its 2 x 2 block
      // and writes the transposed block too
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        if (tk[u] < 0) continue;
        const int k1 = tk[u] & 255, k2 = tk[u] >> 8;
        const f32x4 r1 = ra[u], r2 = rb[u];
        const float c1 = r1[0], s1 = r1[1], c2 = r2[0], s2 = r2[1];
        const int p1 = __float_as_int(r1[2]), q1 = __float_as_int(r1[3]);
        const int p2 = __float_as_int(r2[2]), q2 = __float_as_int(r2[3]);
        const float x00 = T[p1 * TP + p2], x01 = T[p1 * TP + q2];
        const float x10 = T[q1 * TP + p2], x11 = T[q1 * TP + q2];
        const float y00 = c1 * x00 - s1 * x10, y01 = c1 * x01 - s1 * x11;
        const float y10 = s1 * x00 + c1 * x10, y11 = s1 * x01 + c1 * x11;
        float z00 = c2 * y00 - s2 * y01, z01 = s2 * y00 + c2 * y01;
        float z10 = c2 * y10 - s2 * y11, z11 = s2 * y10 + c2 * y11;
        if (k1 == k2 && s1 != 0.f) z01 = z10 = 0.f;
        T[p1 * TP + p2] = z00;
        T[p1 * TP + q2] = z01;
        T[q1 * TP + p2] = z10;
        T[q1 * TP + q2] = z11;
        if (k1 != k2) {
          T[p2 * TP + p1] = z00;
          T[q2 * TP + p1] = z01;
          T[p2 * TP + q1] = z10;
          T[q2 * TP + q1] = z11;
        }
      }
#pragma unroll
      for (int u = 0; u < TE; ++u) {
        if (te[u] < 0) continue;
        const int r0 = te[u] >> 8;
        const f32x4 rk = rc[u];
        if (rk[1] == 0.f) continue;
        f32x4* ep = (f32x4*)(ET + __float_as_int(rk[2]) * EP + r0);
        f32x4* eq = (f32x4*)(ET + __float_as_int(rk[3]) * EP + r0);
        const f32x4 a = *ep, bq = *eq;
        *ep = rk[0] * a - rk[1] * bq;
        *eq = rk[1] * a + rk[0] * bq;
      }
      __syncthreads();
    }
  }
}

template <int D, int LP, bool BATCHED>
__global__ __launch_bounds__(256) void rsvd_mfma_kernel(const PackArgs a) {
  constexpr int kNC = Chunk<LP>::NC, kNRT = Chunk<LP>::NRT;
  using Y = Lay<D, LP>;
  constexpr int NJT = LP / 16;
  constexpr int MAXB = ((LP / 2) * (LP / 2 + 1) / 2 + 255) / 256;  // Gram blocks per thread
  extern __shared__ __align__(16) uint8_t lds[];
  float* ZT = (float*)(lds + Y::zt);
  bf16_t* Ar = (bf16_t*)(lds + Y::x);
  float* CT = (float*)(lds + Y::ct);
  const SmallLay SL = small_lay<D, LP>(min(a.R + a.oversample, D));
  const int GP = SL.jp, TP = SL.tp;
  double* G = (double*)(lds + Y::g);          // pitch GP
  float* Tm = (float*)(lds + Y::g);           // pitch TP
  float* ET = (float*)(lds + SL.et);          // pitch SL.ep
  __shared__ float s_sig[LP];
  __shared__ float s_sinv[LP];
  __shared__ float s_dinv[LP];
  __shared__ int s_perm[LP];
  __shared__ int s_slot[LP];
  __shared__ int s_flag[2];
  __shared__ int s_rflag[2];

  int S = 0, b = 0, g = 0, which = 0, n;
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
    A = (which ? a.V : a.K) + (((int64_t)b * a.L * a.Hkv + (int64_t)a.layer * a.Hkv + g) * a.T + start) * D;
    mat = ((((uint64_t)b * a.L + a.layer) * a.Hkv + g) * 2 + which) * (uint64_t)a.S_max + S;
  }
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = a.R;
  const int l = min(R + a.oversample, min(n, D));

  // ---- orthonormal basis Z of the (approximate) dominant right singular subspace
  if (l < min(n, D)) {
    for (int i = tid; i < LP * D; i += 256) {
      const int j = i / D, d = i - j * D;
      ZT[j * Y::ZP + d] = (j < l) ? gaussian(a.seed, mat, (uint32_t)(d * l + j)) : 0.f;
    }
    __syncthreads();
    for (int it = 0; it <= a.power_iters; ++it) {
      range_step<D, LP>(A, n, lds);
      orthonormalize<D, LP>(lds, l, GP, s_dinv);
    }
  } else if (n <= D) {
    for (int i = tid; i < LP * D; i += 256) {
      const int j = i / D, d = i - j * D;
      ZT[j * Y::ZP + d] = (j < n) ? bfv(A[(int64_t)j * D + d]) : 0.f;
    }
    __syncthreads();
    orthonormalize<D, LP>(lds, l, GP, s_dinv);
    orthonormalize<D, LP>(lds, l, GP, s_dinv);
  } else {
    for (int i = tid; i < LP * D; i += 256) {
      const int j = i / D, d = i - j * D;
      ZT[j * Y::ZP + d] = (j == d && j < l) ? 1.f : 0.f;
    }
    __syncthreads();
  }

  // ---- Rayleigh-Ritz: T = (A Z)^T (A Z)
  {
    const int nb = (l + 1) >> 1, nblk = nb * (nb + 1) / 2;
    double acc[MAXB][4];
#pragma unroll
    for (int i = 0; i < MAXB; ++i) acc[i][0] = acc[i][1] = acc[i][2] = acc[i][3] = 0.0;
    for (int c0 = 0; c0 < n; c0 += kNC) {
      stage<D, kNC, false>(A, n, c0, Ar, nullptr);
      __syncthreads();
      for (int t = wave; t < kNRT * NJT; t += 4) {
        const int rt = t / NJT, jt = t - rt * NJT;
        const f32x4 cv = az_tile<D, 3>(Ar, ZT, rt, jt, lane);
        *(f32x4*)(CT + (jt * 16 + (lane & 15)) * Y::CTP + rt * 16 + 4 * (lane >> 4)) = cv;
      }
      __syncthreads();
#pragma unroll
      for (int bb = 0; bb < MAXB; ++bb) {
        const int t = tid + 256 * bb;
        if (t < nblk) {
          int bj, bi;
          tri_decode(t, bj, bi);
          const float* r0 = CT + 2 * bi * Y::CTP;
          const float* r1 = r0 + Y::CTP;
          const float* q0 = CT + 2 * bj * Y::CTP;
          const float* q1 = q0 + Y::CTP;
          for (int r = 0; r < kNC; r += 4) {
            const f32x4 a0 = *(const f32x4*)(r0 + r), a1 = *(const f32x4*)(r1 + r);
            const f32x4 b0 = *(const f32x4*)(q0 + r), b1 = *(const f32x4*)(q1 + r);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[bb][0] += (double)a0[e] * (double)b0[e];
              acc[bb][1] += (double)a0[e] * (double)b1[e];
              acc[bb][2] += (double)a1[e] * (double)b0[e];
              acc[bb][3] += (double)a1[e] * (double)b1[e];
            }
          }
        }
      }
      __syncthreads();
    }
    for (int i = tid; i < SL.jp * TP; i += 256) Tm[i] = 0.f;
    __syncthreads();
#pragma unroll
    for (int bb = 0; bb < MAXB; ++bb) {
      const int t = tid + 256 * bb;
      if (t < nblk) {
        int bj, bi;
        tri_decode(t, bj, bi);
        const int i0 = 2 * bi, j0 = 2 * bj;
        Tm[i0 * TP + j0] = (float)acc[bb][0]; Tm[j0 * TP + i0] = (float)acc[bb][0];
        Tm[i0 * TP + j0 + 1] = (float)acc[bb][1]; Tm[(j0 + 1) * TP + i0] = (float)acc[bb][1];
        Tm[(i0 + 1) * TP + j0] = (float)acc[bb][2]; Tm[j0 * TP + i0 + 1] = (float)acc[bb][2];
        Tm[(i0 + 1) * TP + j0 + 1] = (float)acc[bb][3]; Tm[(j0 + 1) * TP + i0 + 1] = (float)acc[bb][3];
      }
    }
    __syncthreads();
  }
  // the rotation list follows E^T (the staging region is idle)
  f32x4* s_rot = (f32x4*)(ET + (size_t)SL.jp * SL.ep);
  jacobi<LP>(Tm, ET, l, SL.jp, TP, SL.ep, s_rot, s_rflag);

  // ---- order eigenpairs by decreasing eigenvalue (ties: lower index first)
  for (int i = tid; i < l; i += 256) {
    const float ti = Tm[i * TP + i];
    int rank = 0;
    for (int j = 0; j < l; ++j) {
      const float tj = Tm[j * TP + j];
      rank += (tj > ti) || (tj == ti && j < i);
    }
    s_perm[rank] = i;
  }
  __syncthreads();
  if (tid == 0) {
    const int r = min(R, l);
    const float top = sqrtf(fmaxf(Tm[s_perm[0] * TP + s_perm[0]], 0.f));
    int re = 0;
    for (int i = 0; i < r; ++i) {
      const float sg = sqrtf(fmaxf(Tm[s_perm[i] * TP + s_perm[i]], 0.f));
      const bool keep = sg > 1e-6f * top && sg > 0.f;
      s_sig[i] = keep ? sg : 0.f;
      s_sinv[i] = keep ? 1.f / sg : 0.f;
      re += keep;
    }
    for (int i = r; i < LP; ++i) { s_sig[i] = 0.f; s_sinv[i] = 0.f; }
    s_flag[1] = re;  // leading kept components (eigenvalues are sorted)
  }
  __syncthreads();
  const int re = s_flag[1];

  // ---- V = Z E[:, perm] (D x re) into the rows of ZT; rows re.. are zero
  {
    constexpr int VB = ((D / 4) * (LP / 4) + 255) / 256;
    const int nbi = (re + 3) >> 2;
    const int nvb = (D / 4) * nbi;
    f32x4 v[VB][4];
    int col[VB][4];
#pragma unroll
    for (int bb = 0; bb < VB; ++bb) {
      const int t = tid + 256 * bb;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[bb][e] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < nvb) {
        const int d0 = 4 * (t % (D / 4)), i0 = 4 * (t / (D / 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) col[bb][e] = (i0 + e < re) ? s_perm[i0 + e] : 0;
        for (int k = 0; k < l; ++k) {
          const f32x4 z = *(const f32x4*)(ZT + k * Y::ZP + d0);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[bb][e] += z * ET[col[bb][e] * SL.ep + k];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int bb = 0; bb < VB; ++bb) {
      const int t = tid + 256 * bb;
      if (t < nvb) {
        const int d0 = 4 * (t % (D / 4)), i0 = 4 * (t / (D / 4));
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (i0 + e < re) *(f32x4*)(ZT + (i0 + e) * Y::ZP + d0) = v[bb][e];
      }
    }
    for (int i = tid; i < (LP - re) * D; i += 256) ZT[(re + i / D) * Y::ZP + i % D] = 0.f;
    __syncthreads();
  }

  // ---- U = orth(A V Sigma^-1): Gram of U' (fp64), Cholesky, L^-1, U = U' L^-T
  const int nbu = (re + 1) >> 1, nblku = nbu * (nbu + 1) / 2;
  auto u_chunk = [&](int c0) {
    stage<D, kNC, false>(A, n, c0, Ar, nullptr);
    __syncthreads();
    for (int t = wave; t < kNRT * NJT; t += 4) {
      const int rt = t / NJT, jt = t - rt * NJT;
      f32x4 cv = az_tile<D, 3>(Ar, ZT, rt, jt, lane);
      cv *= s_sinv[jt * 16 + (lane & 15)];
      *(f32x4*)(CT + (jt * 16 + (lane & 15)) * Y::CTP + rt * 16 + 4 * (lane >> 4)) = cv;
    }
    __syncthreads();
  };
  {
    double acc[MAXB][4];
#pragma unroll
    for (int i = 0; i < MAXB; ++i) acc[i][0] = acc[i][1] = acc[i][2] = acc[i][3] = 0.0;
    for (int c0 = 0; c0 < n; c0 += kNC) {
      u_chunk(c0);
#pragma unroll
      for (int bb = 0; bb < MAXB; ++bb) {
        const int t = tid + 256 * bb;
        if (t < nblku) {
          int bj, bi;
          tri_decode(t, bj, bi);
          const float* r0 = CT + 2 * bi * Y::CTP;
          const float* r1 = r0 + Y::CTP;
          const float* q0 = CT + 2 * bj * Y::CTP;
          const float* q1 = q0 + Y::CTP;
          for (int r = 0; r < kNC; r += 4) {
            const f32x4 a0 = *(const f32x4*)(r0 + r), a1 = *(const f32x4*)(r1 + r);
            const f32x4 b0 = *(const f32x4*)(q0 + r), b1 = *(const f32x4*)(q1 + r);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[bb][0] += (double)a0[e] * (double)b0[e];
              acc[bb][1] += (double)a0[e] * (double)b1[e];
              acc[bb][2] += (double)a1[e] * (double)b0[e];
              acc[bb][3] += (double)a1[e] * (double)b1[e];
            }
          }
        }
      }
      if (c0 + kNC < n) __syncthreads();
    }
#pragma unroll
    for (int bb = 0; bb < MAXB; ++bb) {
      const int t = tid + 256 * bb;
      if (t < nblku) {
        int bj, bi;
        tri_decode(t, bj, bi);
        const int i0 = 2 * bi, j0 = 2 * bj;
        G[i0 * GP + j0] = acc[bb][0]; G[j0 * GP + i0] = acc[bb][0];
        G[i0 * GP + j0 + 1] = acc[bb][1]; G[(j0 + 1) * GP + i0] = acc[bb][1];
        G[(i0 + 1) * GP + j0] = acc[bb][2]; G[j0 * GP + i0 + 1] = acc[bb][2];
        G[(i0 + 1) * GP + j0 + 1] = acc[bb][3]; G[(j0 + 1) * GP + i0 + 1] = acc[bb][3];
      }
    }
    __syncthreads();
  }
  cholesky64(G, re, GP, s_dinv);
  // L^-1 (lower), column j by thread j, stored transposed in G's upper triangle:
  // Linv[i][j] at G[j][i] (i > j); Linv[j][j] = dinv[j]
  if (tid < re) {
    const int j = tid;
    const float dj = s_dinv[j];
    for (int i = j + 1; i < re; ++i) {
      float accv = (float)G[i * GP + j] * s_dinv[j] * dj;
      for (int k = j + 1; k < i; ++k) accv += (float)G[i * GP + k] * s_dinv[k] * (float)G[j * GP + k];
      G[j * GP + i] = (double)(-accv * s_dinv[i]);
    }
  }
  __syncthreads();

  // ---- outputs.  Index build: component i is stored in slot s_slot[i] of
  // the blob's rk (K) or rv (V) stored components, in order; a component past
  // min(R, n) or whose gate is below gate_eps is dropped (-1).  Slots past the
  // kept ones stay zero.
  const int npad = Blob::npad(n);
  uint8_t* blob = nullptr;
  int rk = R, rv = R;
  if (!BATCHED) {
    const uint2 ref = a.bref[((int64_t)a.layer * a.Hkv + g) * a.total_spans + bm.span_base + S];
    blob = a.pool + (int64_t)ref.x * 256;
    rk = bref_rk(ref);
    rv = bref_rv(ref);
    if (tid == 0) {
      const int rs = which ? rv : rk;
      const float* gm = a.gates ? a.gates + mat * (int64_t)R : nullptr;   // this matrix's R gates
      int c = 0;
      for (int i = 0; i < R; ++i) {
        const bool k = i < min(R, n) && gate_kept(gm ? gm[i] : 1.f, a.gate_eps) && c < rs;
        s_slot[i] = k ? c++ : -1;
      }
    }
    __syncthreads();
  }
  // right factors and sigma (m)
  if (BATCHED) {
    float* Vo = a.out_Vt + mat * (int64_t)R * D;
    for (int idx = tid; idx < R * D; idx += 256) {
      const int i = idx / D, d = idx - i * D;
      Vo[idx] = (i < re) ? ZT[i * Y::ZP + d] : 0.f;
    }
    for (int i = tid; i < R; i += 256) a.out_S[mat * R + i] = (i < re) ? s_sig[i] : 0.f;
  } else {
    // K -> VKt [rk][D] krow layout, V -> VV [D][rv] a16 layout
    bf16_t* Vo = (bf16_t*)(blob + (which ? Blob::off_vv(rk, D) : Blob::off_vkt()));
    for (int idx = tid; idx < D * re; idx += 256) {
      const int i = idx / D, d = idx - i * D;
      const int sl = s_slot[i];
      if (sl < 0) continue;
      const int64_t o = which ? a16_off(d, sl, rv) : krow_off(sl, d, D);
      Vo[o] = to_bf(ZT[i * Y::ZP + d]);
    }
    float* sm = (float*)(blob + (which ? Blob::off_smv(rk, rv, D) : Blob::off_smk(rk, rv, D)));
    for (int i = tid; i < R; i += 256) {
      const int sl = s_slot[i];
      if (sl < 0) continue;
      const float m = a.gates ? a.gates[mat * (int64_t)R + i] : 1.f;
      sm[sl] = (i < re) ? s_sig[i] * m : 0.f;
    }
  }

  // L^-T as an fp32 table over the G region: Lt[k][i] = Linv[i][k] for
  // k <= i < re, else 0 (read from G into registers, then written over it)
  float* Lt = (float*)G;
  {
    constexpr int NE = (LP * LP + 255) / 256;
    float lt[NE];
#pragma unroll
    for (int c = 0; c < NE; ++c) {
      const int e = tid + 256 * c, k = e / LP, i = e - k * LP;
      lt[c] = (e < LP * LP && i < re && k <= i) ? (k == i ? s_dinv[i] : (float)G[k * GP + i]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NE; ++c)
      if (tid + 256 * c < LP * LP) Lt[tid + 256 * c] = lt[c];
    __syncthreads();
  }

  // ---- U = U' L^-T, one staged chunk of rows at a time: U' as in the Gram
  // pass (the same products, so the same values), then the triangular factor
  // on the fp32 MFMA (16x16x4: A[i][k] and B[k][j] at lane i (j) + 16 k).
  {
    constexpr int NT = (kNRT * NJT + 3) / 4;   // output tiles per wave
    const int kend = (re + 3) & ~3;            // rows re.. of CT and Lt are zero
    for (int c0 = 0; c0 < n; c0 += kNC) {
      u_chunk(c0);
      f32x4 ut[NT];
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        ut[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int t = wave + 4 * q;
        if (t < kNRT * NJT) {
          const int rt = t / NJT, jt = t - rt * NJT;
          for (int k0 = 0; k0 < kend; k0 += 4) {
            const int k = k0 + (lane >> 4);
            const float av = CT[k * Y::CTP + rt * 16 + (lane & 15)];
            const float bv = Lt[k * LP + jt * 16 + (lane & 15)];
            ut[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, ut[q], 0, 0, 0);
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        const int t = wave + 4 * q;
        if (t < kNRT * NJT) {
          const int rt = t / NJT, jt = t - rt * NJT;
          *(f32x4*)(CT + (jt * 16 + (lane & 15)) * Y::CTP + rt * 16 + 4 * (lane >> 4)) = ut[q];
        }
      }
      __syncthreads();
      for (int t = tid; t < kNC * re; t += 256) {
        const int i = t / kNC, r = t - i * kNC;
        const int row = c0 + r;
        if (row >= n) continue;
        const float u = CT[i * Y::CTP + r];
        if (BATCHED) {
          a.out_U[(mat * (int64_t)a.max_rows + row) * R + i] = u;
        } else {
          const int sl = s_slot[i];
          if (sl < 0) continue;
          bf16_t* Uo = (bf16_t*)(blob + (which ? Blob::off_uvt(rk, rv, D, n) : Blob::off_uk(rk, rv, D)));
          Uo[which ? a16_off(sl, row, npad) : a16_off(row, sl, rk)] = to_bf(u);
        }
      }
      __syncthreads();
    }
  }
  if (BATCHED) {
    float* Uo = a.out_U + mat * (int64_t)a.max_rows * R;
    for (int idx = tid; idx < a.max_rows * R; idx += 256) {
      const int row = idx / R, i = idx - row * R;
      if (row >= n || i >= re) Uo[idx] = 0.f;
    }
  }
}

template <int D, int LP, bool BATCHED>
hipError_t launch_lp(const PackArgs& a, dim3 grid, hipStream_t st) {
  const size_t lds = small_lay<D, LP>(min(a.R + a.oversample, D)).bytes;
  hipError_t e = hipFuncSetAttribute((const void*)rsvd_mfma_kernel<D, LP, BATCHED>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rsvd_mfma_kernel<D, LP, BATCHED>), grid, dim3(256), lds, st, a);
  return hipGetLastError();
}

template <bool BATCHED>
hipError_t dispatch(const PackArgs& a, dim3 grid, hipStream_t st) {
  const int lp = (min(a.R + a.oversample, a.D) + 15) & ~15;
  if (a.D == 128) {
    switch (lp) {
      case 16: return launch_lp<128, 16, BATCHED>(a, grid, st);
      case 32: return launch_lp<128, 32, BATCHED>(a, grid, st);
      case 48: return launch_lp<128, 48, BATCHED>(a, grid, st);
      case 64: return launch_lp<128, 64, BATCHED>(a, grid, st);
      case 80: return launch_lp<128, 80, BATCHED>(a, grid, st);
      default: break;
    }
  } else if (a.D == 64) {
    switch (lp) {
      case 16: return launch_lp<64, 16, BATCHED>(a, grid, st);
      case 32: return launch_lp<64, 32, BATCHED>(a, grid, st);
      case 48: return launch_lp<64, 48, BATCHED>(a, grid, st);
      case 64: return launch_lp<64, 64, BATCHED>(a, grid, st);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rsvd(const PackArgs& a, hipStream_t st) {
  if (a.max_spans == 0) return hipSuccess;
  return dispatch<false>(a, dim3(a.max_spans, a.B, a.Hkv * 2), st);
}

hipError_t launch_rsvd_batched(const PackArgs& a, hipStream_t st) {
  if (a.count == 0) return hipSuccess;
  return dispatch<true>(a, dim3(a.count), st);
}

}  // namespace sekv
