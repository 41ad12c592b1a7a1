// Decode attention over the SeKV two-resolution cache, gfx950.
//
// SeKV article (aitrends.kr/articles/75020), section 방법론 (Method), Stage 2
// and Fig. 2: the routed spans are rebuilt to token level from their gated
// factors and merged into the attention output; section 기술 상세 (Technical
// details) gives the reconstruction Khat_S = sum_i m_i sigma_i u_i v_i^T.
//
// One workgroup (4 waves) per work item.  Item j of nj for a KV head (b, g)
// streams a slice of its resident rows (raw tokens, then one pseudo row per
// span) in 32-row steps and takes share j of nj of the union over the G query
// heads of that KV head's routed spans: every item of a launch has the same
// shape, so one launch fits the GPU in a single wave of workgroups and the
// resident loads overlap the span bookkeeping.  For the union share of the
// item's spans the reconstruction is never materialised:
//     t = V^K^T q                    (R)      MFMA 16x16x32, A = V^K^T tile
//     scores = U^K (t . sigma m^K)/sqrt(d)    MFMA 16x16x16, A = U^K tile
//     w = U^V^T p                    (R)      MFMA 16x16x16, A = U^V^T tile
//     o += V^V (sigma m^V . w)       (d)      MFMA 16x16x16, A = V^V tile
// Each product's D operand (lane = head + 16*(row/4)) is the next product's
// B operand, so values never leave registers.  Query heads of the GQA group
// occupy the 16 MFMA columns (G of them live).  fp32 operands that feed a
// bf16 MFMA (softmax weights, scaled t, gated w) are split hi + lo into two
// bf16 terms, which keeps ~16 mantissa bits; every accumulation is fp32.
//
// A span's factor blob, with the second 64-token chunk of its left factors,
// is loaded in one round trip (all its loads issued before any arithmetic;
// V^V and that chunk go to LDS).  Each wave takes its spans longest first,
// from a greedy assignment every wave computes alike from the span lengths,
// so results do not depend on timing.  Each workgroup writes one softmax partial
// (m, l, o) per head; merge_kernel combines them.  (A last-workgroup merge
// inside this kernel would need a device-scope release per workgroup, which
// on this GPU writes back the XCD's L2 each time; the kernel boundary is the
// cheaper synchronisation.)
#include <hip/hip_ext.h>

#include "common.h"

namespace sekv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Loads of the streamed operands (resident rows and factor blobs, each read
// once a step) carry the non-temporal hint when the index is larger than
// the cache can hold across steps (NT), so that they do not push the small
// shared tables (mask words, span metadata, partials) and the next kernels'
// inputs out of L2 and the Infinity Cache (measured 763 -> 775
// query-tokens/s at 128K).  A small index keeps plain loads: its layer stays
// cache-resident from step to step.  The asynchronous loads to LDS take the
// same hint as the cache-policy operand value 2 (the non-temporal bit).
template <int NT, class T>
__device__ __forceinline__ T ld_stream(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load((const T*)p);
  else return *(const T*)p;
}
template <int NT>
constexpr int kLdsStream = NT ? 2 : 0;

__device__ __forceinline__ floatx4 mfma32(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(u32x2 a, u32x2 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a),
                                                   __builtin_bit_cast(short4v, b), c, 0, 0, 0);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ void split2(float x, uint32_t& hi, uint32_t& lo) {
  hi = bf16_bits(x);
  lo = bf16_bits(x - __uint_as_float(hi << 16));
}
__device__ __forceinline__ void pack4(const floatx4 v, u32x2& hi, u32x2& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split2(v[e], h[e], l[e]);
  hi = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  lo = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
}
__device__ __forceinline__ void pack8(const floatx4 a, const floatx4 b, u32x4& hi, u32x4& lo) {
  u32x2 ha, la, hb, lb;
  pack4(a, ha, la);
  pack4(b, hb, lb);
  hi = u32x4{ha[0], ha[1], hb[0], hb[1]};
  lo = u32x4{la[0], la[1], lb[0], lb[1]};
}

__device__ __forceinline__ float xmax4(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float xsum4(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Fold a block of scores (already scaled, masked to -inf) into the running
// softmax state (m, l) of this lane's head and turn them into weights
// relative to the new running max.  Returns the factor by which older
// accumulations must be scaled.
template <int NB>
__device__ __forceinline__ float online(floatx4 (&sc)[NB], int nb, float& m, float& l) {
  float mx = -INFINITY;
#pragma unroll
  for (int tb = 0; tb < NB; ++tb)
    if (tb < nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[tb][r]);
  mx = xmax4(mx);
  const float mnew = fmaxf(m, mx);
  const float corr = (m == -INFINITY) ? 0.f : __expf(m - mnew);
  float ps = 0.f;
#pragma unroll
  for (int tb = 0; tb < NB; ++tb)
    if (tb < nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = sc[tb][r];
        const float p = (x == -INFINITY) ? 0.f : __expf(x - mnew);
        sc[tb][r] = p;
        ps += p;
      }
  ps = xsum4(ps);
  l = l * corr + ps;
  m = mnew;
  return corr;
}

// Registers of one span blob: the fixed-size factors plus the first chunk
// (up to 64 tokens) of the left factors.  V^V, needed only at the end of the
// span, goes to the wave's LDS buffer instead: asynchronous global->LDS loads
// (16 bytes per lane, 1 KB per instruction, lane i's bytes land at 16 i)
// issued with the rest, so it costs no registers and no second round trip.
// The blob holds nrk (nrv) 16-component blocks of key (value) factors, at most
// R / 16 each: the registers are sized for R and the blocks past the stored
// ones are neither loaded nor multiplied (wave-uniform branches).
template <int D, int R, int NT>
struct SpanRegs {
  static constexpr int NS32 = D / 32, ND16 = D / 16, NR16 = R / 16;
  static constexpr int VV_BYTES = 2 * D * R;
  // tokens 64..127 of the left factors (U^K and U^V^T, 4 token blocks each)
  // also go to the wave's LDS with the blob, so a span of up to 128 tokens
  // is one round trip; longer spans stream their further chunks
  static constexpr bool CK = R <= 32;
  static constexpr int CK_BYTES = CK ? 2 * 4 * NR16 * 512 : 16;
  u32x4 vkt[NR16][NS32];
  floatx4 smk[NR16], smv[NR16];
  u32x2 uk[4][NR16];
  u32x2 uvt[NR16][4];
  const uint8_t* blob;
  int n, hm, nrk, nrv;

  __device__ __forceinline__ void load(const uint8_t* b, int n_, int hm_, int ranks, int lane, int grp,
                                       uint8_t* lds_vv, uint8_t* lds_ck) {
    blob = b;
    n = n_;
    hm = hm_;
    // stored ranks rk | rv << 16 (multiples of 16), clamped to [16, R]
    nrk = (NR16 == 1) ? 1 : min(max((ranks & 0xffff) >> 4, 1), NR16);
    nrv = (NR16 == 1) ? 1 : min(max((int)((uint32_t)ranks >> 20), 1), NR16);
    const int rk = 16 * nrk, rv = 16 * nrv;
    const bf16_t* pk = (const bf16_t*)(b + Blob::off_vkt());
    const uint8_t* pv = b + Blob::off_vv(rk, D);
    const float* sk = (const float*)(b + Blob::off_smk(rk, rv, D));
    const float* sv = (const float*)(b + Blob::off_smv(rk, rv, D));
    const bf16_t* pu = (const bf16_t*)(b + Blob::off_uk(rk, rv, D));
    const bf16_t* pw = (const bf16_t*)(b + Blob::off_uvt(rk, rv, D, n_));
    const int ntb = Blob::npad(n_) >> 4;
#pragma unroll
    for (int ib = 0; ib < NR16; ++ib)
      if (ib < nrk)
#pragma unroll
        for (int s = 0; s < NS32; ++s) vkt[ib][s] = ld_stream<NT, u32x4>(pk + ib * 16 * D + s * 512 + lane * 8);
#pragma unroll
    for (int ib = 0; ib < NR16; ++ib) {
      if (ib < nrk) smk[ib] = *(const floatx4*)(sk + 16 * ib + 4 * grp);
      if (ib < nrv) smv[ib] = *(const floatx4*)(sv + 16 * ib + 4 * grp);
    }
    // token blocks past ntb read block ntb - 1 again (in range; never used)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int tbc = min(tb, ntb - 1);
#pragma unroll
      for (int kb = 0; kb < NR16; ++kb)
        if (kb < nrk) uk[tb][kb] = ld_stream<NT, u32x2>(pu + ((int64_t)tbc * nrk + kb) * 256 + lane * 4);
    }
#pragma unroll
    for (int ib = 0; ib < NR16; ++ib)
      if (ib < nrv)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const int tbc = min(tb, ntb - 1);
          uvt[ib][tb] = ld_stream<NT, u32x2>(pw + ((int64_t)ib * ntb + tbc) * 256 + lane * 4);
        }
    // V^V: D rv bf16 = D nrv / 32 KB
#pragma unroll
    for (int c = 0; c < VV_BYTES / 1024; ++c)
      if (c < D * nrv / 32)
        __builtin_amdgcn_global_load_lds((const void*)(pv + c * 1024 + lane * 16),
                                         (__attribute__((address_space(3))) void*)(lds_vv + c * 1024), 16, 0, kLdsStream<NT>);
    if (CK && ntb > 4) {   // wave-uniform
      // 512-byte blocks: U^K (tb, kb) at tb' nrk + kb, then U^V^T (ib, tb) at
      // 4 nrk + 4 ib + tb', tb' = tb - 4; blocks past the span re-read its
      // last block (in range, multiplied by zero weights).  Two blocks a load;
      // nrk is 1 or 2 here (R <= 32), so blk / nrk is a shift.
      const uint8_t* uk8 = (const uint8_t*)pu;
      const uint8_t* uv8 = (const uint8_t*)pw;
      const int sh = nrk - 1;
#pragma unroll
      for (int c = 0; c < 4 * NR16; ++c) {
        if (c < 2 * (nrk + nrv)) {
          const int blk = 2 * c + (lane >> 5);
          int64_t src;
          if (blk < 4 * nrk) {
            const int tb = 4 + (blk >> sh), kb = blk & sh;
            src = (int64_t)(min(tb, ntb - 1) * nrk + kb) * 512;
            src += (int64_t)(uk8 - b);
          } else {
            const int ib = (blk - 4 * nrk) >> 2, tb = 4 + ((blk - 4 * nrk) & 3);
            src = (int64_t)(ib * ntb + min(tb, ntb - 1)) * 512;
            src += (int64_t)(uv8 - b);
          }
          __builtin_amdgcn_global_load_lds((const void*)(b + src + (lane & 31) * 16),
                                           (__attribute__((address_space(3))) void*)(lds_ck + c * 1024), 16, 0, kLdsStream<NT>);
        }
      }
    }
  }
};

// One chunk of up to 64 tokens of a routed span: scores, online softmax and
// the U^V^T p accumulation, over the nrk key and nrv value blocks stored.
template <int D, int G, int R>
__device__ __forceinline__ void span_chunk(const u32x2 (&uk)[4][R / 16], const u32x2 (&uvt)[R / 16][4], int tb0,
                                           int nb, int n, bool act, int grp, int nrk, int nrv,
                                           const u32x2 (&chi)[R / 16], const u32x2 (&clo)[R / 16], float& m,
                                           float& l, floatx4 (&o)[D / 16], floatx4 (&wacc)[R / 16]) {
  constexpr int ND16 = D / 16, NR16 = R / 16;
  floatx4 sc[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    sc[tb] = floatx4{0, 0, 0, 0};
    if (tb < nb) {
#pragma unroll
      for (int kb = 0; kb < NR16; ++kb)
        if (kb < nrk) {
          sc[tb] = mfma16(uk[tb][kb], chi[kb], sc[tb]);
          sc[tb] = mfma16(uk[tb][kb], clo[kb], sc[tb]);
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = 16 * (tb0 + tb) + 4 * grp + r;
        if (!act || tok >= n) sc[tb][r] = -INFINITY;
      }
    }
  }
  const float corr = online<4>(sc, nb, m, l);
#pragma unroll
  for (int db = 0; db < ND16; ++db) o[db] *= corr;
#pragma unroll
  for (int ib = 0; ib < NR16; ++ib) wacc[ib] *= corr;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    if (tb < nb) {
      u32x2 phi, plo;
      pack4(sc[tb], phi, plo);
#pragma unroll
      for (int ib = 0; ib < NR16; ++ib)
        if (ib < nrv) {
          wacc[ib] = mfma16(uvt[ib][tb], phi, wacc[ib]);
          wacc[ib] = mfma16(uvt[ib][tb], plo, wacc[ib]);
        }
    }
  }
}

// Attention over one routed span in factored form, folded into (m, l, o).
template <int D, int G, int R, int NT>
__device__ __forceinline__ void span_pass(const SpanRegs<D, R, NT>& sr, const u32x4 (&qB)[D / 32], float scale,
                                          int lane, int hl, int grp, float& m, float& l,
                                          floatx4 (&o)[D / 16], const uint8_t* lds_vv, const uint8_t* lds_ck) {
  constexpr int NS32 = D / 32, ND16 = D / 16, NR16 = R / 16;
  const int n = sr.n, npad = Blob::npad(n), ntb = npad >> 4;
  const int nrk = sr.nrk, nrv = sr.nrv;
  // t = V^K^T q; c = t * sigma m^K / sqrt(d), split into bf16 hi + lo
  u32x2 chi[NR16], clo[NR16];
#pragma unroll
  for (int ib = 0; ib < NR16; ++ib)
    if (ib < nrk) {
      floatx4 t = floatx4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < NS32; ++s) t = mfma32(sr.vkt[ib][s], qB[s], t);
      pack4(t * sr.smk[ib] * scale, chi[ib], clo[ib]);
    }
  const bool act = (hl < G) && ((sr.hm >> hl) & 1);
  floatx4 wacc[NR16];
#pragma unroll
  for (int ib = 0; ib < NR16; ++ib) wacc[ib] = floatx4{0, 0, 0, 0};
  // first 64 tokens from the preloaded registers, the rest streamed
  span_chunk<D, G, R>(sr.uk, sr.uvt, 0, min(4, ntb), n, act, grp, nrk, nrv, chi, clo, m, l, o, wacc);
  if (ntb > 4) {
    const int rk = 16 * nrk, rv = 16 * nrv;
    const bf16_t* pu = (const bf16_t*)(sr.blob + Blob::off_uk(rk, rv, D));
    const bf16_t* pw = (const bf16_t*)(sr.blob + Blob::off_uvt(rk, rv, D, n));
    for (int tb0 = 4; tb0 < ntb; tb0 += 4) {
      const int nb = min(4, ntb - tb0);
      u32x2 uk[4][NR16], uvt[NR16][4];
      if (SpanRegs<D, R, NT>::CK && tb0 == 4) {
        // from the wave's LDS copy (wait for the wave's outstanding loads,
        // the asynchronous copies included)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
          for (int kb = 0; kb < NR16; ++kb)
            if (kb < nrk) uk[tb][kb] = *(const u32x2*)(lds_ck + (tb * nrk + kb) * 512 + lane * 8);
#pragma unroll
          for (int ib = 0; ib < NR16; ++ib)
            if (ib < nrv) uvt[ib][tb] = *(const u32x2*)(lds_ck + (4 * nrk + ib * 4 + tb) * 512 + lane * 8);
        }
      } else {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const int tbc = tb0 + min(tb, nb - 1);
#pragma unroll
          for (int kb = 0; kb < NR16; ++kb)
            if (kb < nrk) uk[tb][kb] = ld_stream<NT, u32x2>(pu + ((int64_t)tbc * nrk + kb) * 256 + lane * 4);
#pragma unroll
          for (int ib = 0; ib < NR16; ++ib)
            if (ib < nrv) uvt[ib][tb] = ld_stream<NT, u32x2>(pw + ((int64_t)ib * ntb + tbc) * 256 + lane * 4);
        }
      }
      span_chunk<D, G, R>(uk, uvt, tb0, nb, n, act, grp, nrk, nrv, chi, clo, m, l, o, wacc);
    }
  }
  // o += V^V (sigma m^V . w)
  u32x2 whi[NR16], wlo[NR16];
#pragma unroll
  for (int ib = 0; ib < NR16; ++ib)
    if (ib < nrv) pack4(wacc[ib] * sr.smv[ib], whi[ib], wlo[ib]);
  // V^V from the wave's LDS copy: wait for every outstanding load of the
  // wave, the asynchronous copies included
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const bf16_t* pv = (const bf16_t*)lds_vv;
#pragma unroll
  for (int db = 0; db < ND16; ++db)
#pragma unroll
    for (int kb = 0; kb < NR16; ++kb)
      if (kb < nrv) {
        const u32x2 vvv = *(const u32x2*)(pv + ((db * nrv + kb) * 256 + lane * 4));
        o[db] = mfma16(vvv, whi[kb], o[db]);
        o[db] = mfma16(vvv, wlo[kb], o[db]);
      }
}

// One 32-row step of resident rows for the lane's head: two 16-row key
// blocks, one 32-row value block, and for pseudo rows the head's mask bit
// and the ln n_S bias, all loaded in one round trip (branch-free: clamped
// in-range loads, invalid rows masked afterwards).  Every global load from
// here to the first fold is issued without a branch: the wait before the
// fold then counts only the loads issued after this step's, which stay in
// flight.
template <int D, int G, int NT>
struct ResStep {
  static constexpr int NS32 = D / 32, ND16 = D / 16;
  u32x4 kt[2][NS32], vt[ND16];
  uint32_t word[2][4];   // the 32-bit half of the mask word holding the row's bit
  float lgn[2][4];
  int t;

  __device__ __forceinline__ void load(const bf16_t* Kb, const bf16_t* Vb, const uint64_t* mh, const float* logn,
                                       const BMeta& bm, int t_, int lane, int grp) {
    t = t_;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < NS32; ++s)
        kt[kb][s] = ld_stream<NT, u32x4>(Kb + (int64_t)(2 * t + kb) * 16 * D + s * 512 + lane * 8);
#pragma unroll
    for (int db = 0; db < ND16; ++db) vt[db] = ld_stream<NT, u32x4>(Vb + (int64_t)t * 32 * D + db * 512 + lane * 8);
    // pseudo-row inputs, loaded for every step (no branch, so that later
    // waits can count these loads); raw rows read span 0 and are masked
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sp = 32 * t + 16 * kb + 4 * grp + r - bm.n_raw;
        const int spc = max(min(sp, bm.n_spans - 1), 0);
        word[kb][r] = ((const uint32_t*)mh)[spc >> 5];
        lgn[kb][r] = logn[bm.n_spans > 0 ? bm.span_base + spc : 0];
      }
  }

  // scores, online softmax and o += V p for this step
  __device__ __forceinline__ void fold(const u32x4 (&qB)[NS32], const BMeta& bm, float scale, int hl, int grp,
                                       float& m, float& l, floatx4 (&o)[ND16]) const {
    const int row0 = 32 * t;
    const bool has_pseudo = row0 + 32 > bm.n_raw && bm.n_spans > 0;
    floatx4 S[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      S[kb] = floatx4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < NS32; ++s) S[kb] = mfma32(kt[kb][s], qB[s], S[kb]);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 16 * kb + 4 * grp + r;
        float x = S[kb][r] * scale;
        if (hl >= G || row >= bm.n_res) x = -INFINITY;
        else if (has_pseudo && row >= bm.n_raw) {
          // a span expanded by this head is attended through its factors
          const int sp = row - bm.n_raw;
          x = ((word[kb][r] >> (sp & 31)) & 1u) ? -INFINITY : x + lgn[kb][r];
        }
        S[kb][r] = x;
      }
    const float corr = online<2>(S, 2, m, l);
#pragma unroll
    for (int db = 0; db < ND16; ++db) o[db] *= corr;
    u32x4 phi, plo;
    pack8(S[0], S[1], phi, plo);
#pragma unroll
    for (int db = 0; db < ND16; ++db) {
      o[db] = mfma32(vt[db], phi, o[db]);
      o[db] = mfma32(vt[db], plo, o[db]);
    }
  }
};

// Wave-wide sum, and inclusive prefix over lanes, of per-lane counts below
// 2^11, by bit-sliced ballots (scalar popcounts, no lane-to-lane moves).
__device__ __forceinline__ int wave_sum_small(int c) {
  int s = 0;
#pragma unroll
  for (int i = 0; i < 11; ++i) s += (int)__popcll(__ballot((c >> i) & 1)) << i;
  return s;
}
__device__ __forceinline__ int wave_prefix_small(int c, int lane, int& total) {
  const uint64_t le = (2ull << lane) - 1;   // lanes <= lane (all 64 for lane 63)
  int s = 0, t = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) {   // counts of one mask word: at most 64
    const uint64_t bal = __ballot((c >> i) & 1);
    s += (int)__popcll(bal & le) << i;
    t += (int)__popcll(bal) << i;
  }
  total = t;
  return s;
}

// Dynamic LDS of attend_kernel: the union of the G heads' mask words, then
// the G heads' words, [(G + 1)][W] uint64.
inline size_t attend_dyn_lds(int G, int W) { return (size_t)(G + 1) * W * sizeof(uint64_t); }

// Work split of the merge: DSPLIT workgroups per (b, g), each taking DS of
// the D dims of all G heads, NPL outputs per lane.  A partial (one work
// item's G heads) is stored as o[DSPLIT][G][DS] followed by (m, l) of each
// head, so that a merge workgroup reads its slice of every head as one
// contiguous run and the (m, l) of all heads from one line.
template <int D, int G>
struct MergeShape {   // lane layout of the merge
  static constexpr int DSPLIT = (G * D >= 64) ? G * D / 64 : 1;
  static constexpr int DS = D / DSPLIT;            // dims per workgroup
  static constexpr int NPL = G * DS / 64;          // outputs per lane (1 or 2)
};

template <int D, int G, int R, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(R <= 16 ? 3 : (R <= 32 ? 2 : 1))))
void attend_kernel(const AttendArgs a) {
  constexpr int NS32 = D / 32, ND16 = D / 16;
  static_assert(G >= 1 && G <= 16, "G");
  __shared__ float s_ml[4][2][G];
  __shared__ float s_o[4][G][D];
  // per wave: the item's share of the union (span id | active heads << 24
  // by rank within the share), then the wave's own spans in the order it
  // takes them: blob offset, length, active heads, stored ranks
  __shared__ int32_t s_ln[4][kMaxSpanList];
  __shared__ int64_t s_woff[4][kMaxSpanList];
  __shared__ int32_t s_wn[4][kMaxSpanList];
  __shared__ int32_t s_wr[4][kMaxSpanList];   // stored ranks rk | rv << 16
  __shared__ __attribute__((aligned(16))) uint8_t s_vv[4][SpanRegs<D, R, NT>::VV_BYTES];   // per wave
  __shared__ __attribute__((aligned(16))) uint8_t s_ck[4][SpanRegs<D, R, NT>::CK_BYTES];   // per wave
  extern __shared__ uint64_t s_dyn[];

  const WorkItem it = a.items[blockIdx.x];
  const int lc = a.lc_first + blockIdx.y, l = a.layer_begin + lc;
  const int b = it.b, g = it.g;
  const BMeta bm = a.meta[b];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hl = lane & 15, grp = lane >> 4;
  const int Hq = a.Hq, Wd = a.W;
  uint64_t* s_uw = s_dyn;        // [Wd] union words
  uint64_t* s_hw = s_dyn + Wd;   // [G][Wd] head words

  // query operand: B[k = dim][j = head] (lanes of absent heads load head 0
  // and zero it)
  u32x4 qB[NS32];
  {
    const bf16_t* qp = a.q + (((int64_t)b * a.layer_count + lc) * Hq + g * G + (hl < G ? hl : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS32; ++s) {
      const u32x4 v = *(const u32x4*)(qp + 32 * s + 8 * grp);
      qB[s] = (hl < G) ? v : u32x4{0, 0, 0, 0};
    }
  }
  const uint64_t* mrow = a.mask + (((int64_t)b * a.layer_count + lc) * Hq + g * G) * Wd;
  const bool spans = bm.n_spans > 0;   // uniform

  // running softmax state of this lane's head hl; o[dim = 16*db + 4*grp + r]
  float m = -INFINITY, lsum = 0.f;
  floatx4 o[ND16];
#pragma unroll
  for (int db = 0; db < ND16; ++db) o[db] = floatx4{0, 0, 0, 0};
  const float scale = a.scale;

  // the G heads' mask words of word threadIdx.x (more words below)
  const int w0 = min((int)threadIdx.x, Wd - 1);
  uint64_t mw[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mw[h] = mrow[(int64_t)h * Wd + w0];

  // resident slice: wave w takes steps step_begin + w, + 4, ...; the first
  // one's loads stay in flight during the span bookkeeping below
  const int64_t lg = (int64_t)l * a.Hkv + g;
  // start of layer l's blobs in `pool`
  const int64_t lbase = a.layer_off[l] - a.layer_off[a.pool_layer0];
  const bf16_t* Kb = a.kres + bm.res_base + lg * bm.n_res_pad * D;
  const bf16_t* Vb = a.vres + bm.res_base + lg * bm.n_res_pad * D;
  const uint64_t* mh = mrow + (int64_t)(hl < G ? hl : 0) * Wd;
  int t = it.step_begin + wave;
  ResStep<D, G, NT> rs;
  rs.load(Kb, Vb, mh, a.logn, bm, (it.step_begin < it.step_end) ? min(t, it.step_end - 1) : 0, lane, grp);

  // union of the G heads' mask words (bits at or past N_S(b) ignored,
  // whatever the caller's mask holds) and the heads' words, in LDS
  auto put_word = [&](int w, const uint64_t (&x)[G]) {
    const int left = bm.n_spans - 64 * w;
    const uint64_t valid = left >= 64 ? ~0ull : (left > 0 ? (1ull << left) - 1 : 0ull);
    uint64_t u = 0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_hw[h * Wd + w] = x[h] & valid;
      u |= x[h] & valid;
    }
    s_uw[w] = u;
  };
  put_word(w0, mw);   // threads past Wd rewrite word Wd - 1 with the same values
  for (int w = threadIdx.x + 256; w < Wd; w += 256) {
    uint64_t x[G];
#pragma unroll
    for (int h = 0; h < G; ++h) x[h] = mrow[(int64_t)h * Wd + w];
    put_word(w, x);
  }
  __syncthreads();

  // every wave: union size U, the item's ranks [b0, b1) = share j of nj, and
  // the spans of those ranks (a ballot picks the words that overlap the
  // share, each lane places the bit of its own position); lane k then holds
  // the share's k-th span: id | active heads << 24, length, blob offset
  int U = 0;
  for (int w = lane; w < Wd; w += 64) U += __popcll(s_uw[w]);
  U = wave_sum_small(U);
  // 32-bit: the plan keeps nj * N_S below 2^31
  const int b0 = spans ? (int)((uint32_t)it.j * (uint32_t)U / (uint32_t)it.nj) : 0;
  const int b1 = spans ? min((int)((uint32_t)(it.j + 1) * (uint32_t)U / (uint32_t)it.nj), b0 + kMaxSpanList) : 0;
  const int nsh = b1 - b0;
  {
    int carry = 0;
    for (int base = 0; base < Wd && carry < b1; base += 64) {
      const int w = base + lane;
      const uint64_t u = (w < Wd) ? s_uw[w] : 0ull;
      const int c = __popcll(u);
      int tot;
      const int pre = carry + wave_prefix_small(c, lane, tot) - c;
      uint64_t hit = __ballot(c > 0 && pre < b1 && pre + c > b0);
      while (hit) {
        const int src = __builtin_ctzll(hit);
        hit &= hit - 1;
        const int ww = base + src;
        const uint32_t ulo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, src);
        const uint32_t uhi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), src);
        const uint64_t uw = ((uint64_t)uhi << 32) | ulo;
        const int r = __builtin_amdgcn_readlane(pre, src) + (int)__popcll(uw & ((1ull << lane) - 1));
        if (((uw >> lane) & 1ull) && r >= b0 && r < b1) {
          int hm = 0;
#pragma unroll
          for (int h = 0; h < G; ++h) hm |= (int)((s_hw[h * Wd + ww] >> lane) & 1ull) << h;
          s_ln[wave][r - b0] = (64 * ww + lane) | (hm << 24);
        }
      }
      carry += tot;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // (clamped, branch-free: a lane past the share, or an empty share, reads a
  // valid span and is ignored)
  const int ek = (nsh > 0) ? s_ln[wave][min(lane, nsh - 1)] : 0;
  const int Sk = spans ? bm.span_base + (ek & 0xffffff) : 0;
  const int nk = a.span_len[Sk];
  const uint2 rfk = a.bref[lg * a.total_spans + Sk];
  const int64_t ok = lbase + (int64_t)rfk.x * 256;

  // resident slice: fold (the span metadata loads are in flight)
  if (t < it.step_end) {
    rs.fold(qB, bm, scale, hl, grp, m, lsum, o);
    for (t += 4; t < it.step_end; t += 4) {
      rs.load(Kb, Vb, mh, a.logn, bm, t, lane, grp);
      rs.fold(qB, bm, scale, hl, grp, m, lsum, o);
    }
  }

  // routed spans: longest first, each to the wave with the least work so far
  // (greedy LPT; cost in round trips: the blob with its first 64 tokens, one
  // per further 64 tokens, and one for the compute).  Every wave computes the
  // same assignment from the lengths alone, so results do not depend on
  // timing.
  if (nsh > 0) {
    const int nv = (lane < nsh) ? nk : -1;
    int rank = 0;
    for (int j = 0; j < nsh; ++j) {
      const int nj = __builtin_amdgcn_readlane(nv, j);
      rank += (nj > nv) || (nj == nv && j < lane);
    }
    int er = 0;   // lane r: the share index of the rank-r span
    for (int j = 0; j < nsh; ++j) er = (__builtin_amdgcn_readlane(rank, j) == lane) ? j : er;
    const int cr = 1 + (__shfl(nv, er) + 63) / 64;
    int load0 = 0, load1 = 0, load2 = 0, load3 = 0, wr = 0;
    for (int r = 0; r < nsh; ++r) {
      const int c = __builtin_amdgcn_readlane(cr, r);
      int w = 0, lw = load0;
      if (load1 < lw) { w = 1; lw = load1; }
      if (load2 < lw) { w = 2; lw = load2; }
      if (load3 < lw) { w = 3; lw = load3; }
      if (w == 0) load0 += c; else if (w == 1) load1 += c; else if (w == 2) load2 += c; else load3 += c;
      if (lane == r) wr = w;
    }
    // this wave's spans, longest first, into its LDS list
    const uint64_t mine = __ballot(lane < nsh && wr == wave);
    const uint32_t olo = __shfl((uint32_t)ok, er), ohi = __shfl((uint32_t)((uint64_t)ok >> 32), er);
    const int ne = __shfl(nk, er), he = (int)((uint32_t)__shfl(ek, er) >> 24);
    const int rke = __shfl((int)rfk.y, er);
    if ((mine >> lane) & 1ull) {
      const int pos = (int)__popcll(mine & ((1ull << lane) - 1));
      s_woff[wave][pos] = (int64_t)(((uint64_t)ohi << 32) | olo);
      s_wn[wave][pos] = ne | (he << 24);
      s_wr[wave][pos] = rke;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int nw = (int)__popcll(mine);
    for (int i = 0; i < nw; ++i) {
      const int nh = s_wn[wave][i];
      SpanRegs<D, R, NT> cur;
      cur.load(a.pool + uni64(s_woff[wave][i]), uni(nh & 0xffffff), uni((int)((uint32_t)nh >> 24)),
               uni(s_wr[wave][i]), lane, grp, s_vv[wave], s_ck[wave]);
      span_pass<D, G, R, NT>(cur, qB, scale, lane, hl, grp, m, lsum, o, s_vv[wave], s_ck[wave]);
    }
  }

  // ------------------------------------------- merge the 4 waves, write partial
  if (hl < G) {
    if (grp == 0) {
      s_ml[wave][0][hl] = m;
      s_ml[wave][1][hl] = lsum;
    }
#pragma unroll
    for (int db = 0; db < ND16; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_o[wave][hl][16 * db + 4 * grp + r] = o[db][r];
  }
  __syncthreads();
  const int64_t pstride = (int64_t)G * (D + 2);
  float* part = a.part + ((int64_t)lc * a.n_items + it.slot) * pstride;
  constexpr int DS = MergeShape<D, G>::DS;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {   // idx: position in o[DSPLIT][G][DS]
    const int zs = idx / (G * DS), rem = idx - zs * (G * DS);
    const int h = rem / DS, dim = zs * DS + (rem - h * DS);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_ml[w][0][h]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_ml[w][0][h];
      const float e = (mw == -INFINITY) ? 0.f : __expf(mw - M);
      O += e * s_o[w][h][dim];
      L += e * s_ml[w][1][h];
    }
    part[idx] = O;
    if (dim == 0) {
      part[G * D + 2 * h] = M;
      part[G * D + 2 * h + 1] = L;
    }
  }

}

// Merge the partials of every item of (b, g) into out[b][lc][h][:].  Each
// workgroup takes one slice of D / DSPLIT dims for all G heads, one output
// per lane (64 outputs a workgroup: twice the workgroups of two a lane,
// measured 0.4 us faster per 128K layer); each wave folds a quarter of the
// partials into a running (max, denominator, sum) with every load of a
// 24-partial chunk issued before any use, and the four wave states are
// combined in LDS.  grid (B * Hkv * DSPLIT, Lc).

template <int D, int G>
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
  using MS = MergeShape<D, G>;
  constexpr int DS = MS::DS, NPL = MS::NPL;
  constexpr int CH = 24;                       // partials per wave per round trip (2 loads each:
                                               // at most 63 loads in flight per wave)
  static_assert(NPL == 1 || NPL == 2, "merge lane layout");
  __shared__ float s_o[4][G * DS];
  __shared__ float s_m[4][G], s_l[4][G];
  const int bg = blockIdx.x / MS::DSPLIT, z = blockIdx.x - bg * MS::DSPLIT, lc = blockIdx.y;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int first = a.bg_first[2 * bg];
  const int P = a.bg_first[2 * bg + 1];
  const int64_t pstride = (int64_t)G * (D + 2);
  const float* base = a.part + ((int64_t)lc * a.n_items + first) * pstride;
  const int o0 = lane * NPL, h = o0 / DS;   // this lane: head h, dim z * DS + o0 - h * DS
  // online merge over this wave's partials i = wave (mod 4), CH at a time
  float M = -INFINITY, L = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int c0 = wave; c0 < P; c0 += 4 * CH) {
    float mv[CH], lv[CH], v0[CH], v1[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      // branch-free: partials past P re-read partial P - 1 and are ignored
      const int i = c0 + 4 * c;
      const bool ok = i < P;
      const float* p = base + min(i, P - 1) * pstride;
      const float2 ml = *(const float2*)(p + G * D + 2 * h);
      mv[c] = ok ? ml.x : -INFINITY;
      lv[c] = ok ? ml.y : 0.f;
      const float* po = p + z * (G * DS) + o0;   // this workgroup's slice, lane o0
      if (NPL == 2) {
        const float2 v = *(const float2*)po;
        v0[c] = ok ? v.x : 0.f;
        v1[c] = ok ? v.y : 0.f;
      } else {
        v0[c] = ok ? po[0] : 0.f;
        v1[c] = 0.f;
      }
    }
    float mx = M;
#pragma unroll
    for (int c = 0; c < CH; ++c) mx = fmaxf(mx, mv[c]);
    const float corr = (M == -INFINITY) ? 0.f : __expf(M - mx);
    L *= corr;
    acc0 *= corr;
    acc1 *= corr;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const float e = (mv[c] == -INFINITY) ? 0.f : __expf(mv[c] - mx);
      L += e * lv[c];
      acc0 += e * v0[c];
      acc1 += e * v1[c];
    }
    M = mx;
  }
  // combine the four waves
  if ((o0 - h * DS) == 0) {
    s_m[wave][h] = M;
    s_l[wave][h] = L;
  }
  __syncthreads();
  float Mt = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) Mt = fmaxf(Mt, s_m[w][h]);
  const float sc = (M == -INFINITY) ? 0.f : __expf(M - Mt);
  s_o[wave][o0] = acc0 * sc;
  if (NPL == 2) s_o[wave][o0 + 1] = acc1 * sc;
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * DS; idx += 256) {
    const int hh = idx / DS, dd = z * DS + (idx - hh * DS);
    float Mh = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mh = fmaxf(Mh, s_m[w][hh]);
    float Lh = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_m[w][hh];
      Lh += (mw == -INFINITY) ? 0.f : __expf(mw - Mh) * s_l[w][hh];
    }
    const float O = s_o[0][idx] + s_o[1][idx] + s_o[2][idx] + s_o[3][idx];
    a.out[(((int64_t)b * a.layer_count + lc) * a.Hq + g * G + hh) * D + dd] = (Lh > 0.f) ? O / Lh : 0.f;
  }
}

// ------------------------------------------------------------- dispatch
#define SEKV_FOR_R(D, G)                                                     \
  if (R == 16) return f(std::integral_constant<int, D>{}, std::integral_constant<int, G>{}, std::integral_constant<int, 16>{}); \
  if (R == 32) return f(std::integral_constant<int, D>{}, std::integral_constant<int, G>{}, std::integral_constant<int, 32>{}); \
  if (R == 64 && D >= 64) return f(std::integral_constant<int, D>{}, std::integral_constant<int, G>{}, std::integral_constant<int, 64>{});

#define SEKV_FOR_G(D)   \
  if (G == 1) { SEKV_FOR_R(D, 1) } \
  if (G == 2) { SEKV_FOR_R(D, 2) } \
  if (G == 4) { SEKV_FOR_R(D, 4) } \
  if (G == 8) { SEKV_FOR_R(D, 8) }

template <class F>
static hipError_t dispatch(int D, int G, int R, F f) {
  if (D == 64) { SEKV_FOR_G(64) }
  if (D == 128) { SEKV_FOR_G(128) }
  return hipErrorInvalidValue;
}

bool attend_supported(int D, int G, int R) {
  return (D == 64 || D == 128) && (G == 1 || G == 2 || G == 4 || G == 8) &&
         (R == 16 || R == 32 || R == 64) && R <= D;
}

// Every instance the dispatch below can select, instantiated explicitly so
// that each one's device code and host handle are emitted.
#define SEKV_INST_ATTEND(D, G, R)                                        \
  template __global__ void attend_kernel<D, G, R, 0>(const AttendArgs); \
  template __global__ void attend_kernel<D, G, R, 1>(const AttendArgs);
#define SEKV_INST_ATTEND_G(D, G) SEKV_INST_ATTEND(D, G, 16) SEKV_INST_ATTEND(D, G, 32) SEKV_INST_ATTEND(D, G, 64)
SEKV_INST_ATTEND_G(64, 1) SEKV_INST_ATTEND_G(64, 2) SEKV_INST_ATTEND_G(64, 4) SEKV_INST_ATTEND_G(64, 8)
SEKV_INST_ATTEND_G(128, 1) SEKV_INST_ATTEND_G(128, 2) SEKV_INST_ATTEND_G(128, 4) SEKV_INST_ATTEND_G(128, 8)
#undef SEKV_INST_ATTEND_G
#undef SEKV_INST_ATTEND

// Host handles of the two streaming flavours of the attention kernel for
// (D, G, R): [0] plain loads, [1] non-temporal.  Every host use goes through
// this one place that names each instance (a kernel instance named from a
// second host function template failed to compile or to link with this
// toolchain).
struct AttendKernels {
  const void* fn[2];
};
AttendKernels attend_kernels(int D, int G, int R) {
  AttendKernels out{{nullptr, nullptr}};
  (void)dispatch(D, G, R, [&](auto d_, auto g_, auto r_) -> hipError_t {
    constexpr int D_ = decltype(d_)::value, G_ = decltype(g_)::value, R_ = decltype(r_)::value;
    auto cached = attend_kernel<D_, G_, R_, 0>;
    auto streamed = attend_kernel<D_, G_, R_, 1>;
    out.fn[0] = (const void*)cached;
    out.fn[1] = (const void*)streamed;
    return hipSuccess;
  });
  return out;
}

hipError_t attend_slots(int D, int G, int R, int W, int device, int* slots) {
  *slots = 0;
  const AttendKernels k = attend_kernels(D, G, R);
  if (!k.fn[1]) return hipErrorInvalidValue;
  // both flavours use the same registers and LDS
  int per_cu = 0, cus = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k.fn[1], 256, attend_dyn_lds(G, W));
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return e;
  *slots = per_cu * cus;
  return hipSuccess;
}

hipError_t launch_merge(const MergeArgs& a, int D, int G, hipStream_t st) {
  return dispatch(D, G, 16, [&](auto d_, auto g_, auto) -> hipError_t {
    constexpr int D_ = decltype(d_)::value, G_ = decltype(g_)::value;
    hipLaunchKernelGGL((merge_kernel<D_, G_>), dim3(a.B * a.Hkv * MergeShape<D_, G_>::DSPLIT, a.layer_count),
                       dim3(256), 0, st, a);
    return hipGetLastError();
  });
}

hipError_t launch_attend(const AttendArgs& a, int D, int G, int R, hipStream_t st, hipEvent_t ev_start,
                         hipEvent_t ev_stop) {
  if (a.W > 1024 || a.lc_first < 0 || a.lc_count < 1 || a.lc_first + a.lc_count > a.layer_count)
    return hipErrorInvalidValue;
  size_t fixed = 0;
  const hipError_t e0 = dispatch(D, G, R, [&](auto d_, auto g_, auto r_) -> hipError_t {
    constexpr int D_ = decltype(d_)::value, G_ = decltype(g_)::value, R_ = decltype(r_)::value;
    fixed = sizeof(float) * (4 * 2 * G_ + 4 * G_ * D_) + 4 * 20 * kMaxSpanList +
            4 * (SpanRegs<D_, R_, 1>::VV_BYTES + SpanRegs<D_, R_, 1>::CK_BYTES);
    return hipSuccess;
  });
  if (e0 != hipSuccess) return e0;
  const size_t dyn = attend_dyn_lds(G, a.W);
  if (fixed + dyn > 160 * 1024) return hipErrorInvalidValue;
  const void* kern = attend_kernels(D, G, R).fn[a.stream ? 1 : 0];
  if (!kern) return hipErrorInvalidValue;
  if (dyn > 32 * 1024) {
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
  }
  AttendArgs arg = a;
  void* args[] = {&arg};
  if (ev_start)
    return hipExtLaunchKernel(kern, dim3(a.n_items, a.lc_count), dim3(256), args, dyn, st, ev_start, ev_stop, 0);
  return hipLaunchKernel(kern, dim3(a.n_items, a.lc_count), dim3(256), args, dyn, st);
}

}  // namespace sekv
