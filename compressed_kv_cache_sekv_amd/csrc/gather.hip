// Pinned-host factor tier: gather the routed spans' factor blobs into the HBM
// staging ring, gfx950.
//
// SeKV article (aitrends.kr/articles/75020), section 방법론 (Method): the span
// factors live in CPU memory and, for the spans the router expands, U, Sigma
// and V are transferred asynchronously to the GPU before reconstruction;
// section 한계점 (Limitations): this CPU-GPU bandwidth is the method's stated
// cost.
//
// The pinned pool is mapped into the device address space and read by the
// kernel over PCIe.  The HBM ring mirrors the pool's layout for the layers of
// one launch (layer l's region at layer_off[l] - layer_off[ring_layer0]): a blob
// lands at its own offset within its layer's region, so no placement is
// computed on the host and the call does not synchronise.  Blobs hold only the
// components the build kept, so a smaller effective rank moves fewer bytes.  gather_kernel, per (layer, b, KV head, share):
// forms the union over the G heads' masks and its rank and byte prefix per
// mask word, and copies its share of the union's blobs; share 0 records the
// union's size for the call's statistics.
#include "common.h"

namespace sekv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t valid_bits(int n_spans, int w) {
  const int left = n_spans - 64 * w;
  return left >= 64 ? ~0ull : (left > 0 ? (1ull << left) - 1 : 0ull);
}

constexpr int kShare = 128;   // union spans one gather workgroup copies

__global__ __launch_bounds__(256) void gather_kernel(const GatherArgs a) {
  __shared__ uint64_t s_uw[kMaxWords];
  __shared__ int32_t s_pre[kMaxWords + 1];      // union spans before word w
  __shared__ int64_t s_bpre[kMaxWords + 1];     // union bytes before word w
  __shared__ int64_t s_src[kShare];             // blob byte offset within the layer
  __shared__ int32_t s_len[kShare];             // 16-byte chunks
  const int li = a.lc_first + blockIdx.y, l = a.layer_begin + li;
  const int j = blockIdx.x % a.nsplit, bg = blockIdx.x / a.nsplit;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const BMeta bm = a.meta[b];
  const int64_t rid = ((int64_t)li * a.B + b) * a.Hkv + g;
  const uint64_t* mrow = a.mask + (((int64_t)b * a.layer_count + li) * a.Hq + (int64_t)g * a.G) * a.W;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // blob references of (l, g) for b's spans
  const uint2* bref = a.bref + ((int64_t)l * a.Hkv + g) * a.total_spans + bm.span_base;
  const int32_t* slen = a.span_len + bm.span_base;
  for (int w = threadIdx.x; w < a.W; w += 256) {
    uint64_t u = 0;
    for (int h = 0; h < a.G; ++h) u |= mrow[(int64_t)h * a.W + w];
    u &= valid_bits(bm.n_spans, w);
    s_uw[w] = u;
    int64_t by = 0;
    for (uint64_t v = u; v; v &= v - 1) {
      const int S = 64 * w + __builtin_ctzll(v);
      const uint2 r = bref[S];
      by += Blob::bytes(bref_rk(r), bref_rv(r), a.D, slen[S]);
    }
    s_bpre[w + 1] = by;
    s_pre[w + 1] = __popcll(u);
  }
  __syncthreads();
  if (wave == 0) {   // inclusive scans of the per-word counts and bytes
    int carry = 0;
    int64_t bcarry = 0;
    for (int base = 0; base < a.W; base += 64) {
      const int w = base + lane;
      int v = (w < a.W) ? s_pre[w + 1] : 0;
      int64_t by = (w < a.W) ? s_bpre[w + 1] : 0;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(v, d);
        const int64_t yb = __shfl_up(by, d);
        if (lane >= d) {
          v += y;
          by += yb;
        }
      }
      if (w < a.W) {
        s_pre[w + 1] = carry + v;
        s_bpre[w + 1] = bcarry + by;
      }
      carry += __shfl(v, 63);
      bcarry += __shfl(by, 63);
    }
    if (lane == 0) {
      s_pre[0] = 0;
      s_bpre[0] = 0;
    }
  }
  __syncthreads();
  const int U = s_pre[a.W];
  if (j == 0 && threadIdx.x == 0 && a.stat) a.stat[rid] = make_int2(U, (int)(s_bpre[a.W] >> 8));
  const int beg = (int)((int64_t)j * U / a.nsplit), end = (int)((int64_t)(j + 1) * U / a.nsplit);
  const int cnt = min(end - beg, kShare);   // the host keeps shares <= kShare
  // this share's blobs: offset within the layer and 16-byte chunks
  for (int w = threadIdx.x; w < a.W; w += 256) {
    int k = s_pre[w];
    if (k >= beg + cnt || s_pre[w + 1] <= beg) continue;
    for (uint64_t u = s_uw[w]; u && k < beg + cnt; u &= u - 1) {
      const int S = 64 * w + __builtin_ctzll(u);
      if (k >= beg) {
        const uint2 r = bref[S];
        s_src[k - beg] = (int64_t)r.x * 256;
        s_len[k - beg] = (int32_t)(Blob::bytes(bref_rk(r), bref_rv(r), a.D, slen[S]) >> 4);
      }
      ++k;
    }
  }
  __syncthreads();
  // copy to the same offset of ring layer li, 16 bytes per lane, four loads
  // in flight per lane
  const uint8_t* src_l = a.host_pool + a.layer_off[l];
  uint8_t* dst_l = a.ring + (a.layer_off[l] - a.layer_off[a.ring_layer0]);
  for (int e = 0; e < cnt; ++e) {
    const u32x4* src = (const u32x4*)(src_l + s_src[e]);
    u32x4* dst = (u32x4*)(dst_l + s_src[e]);
    const int nch = s_len[e];
    for (int c0 = threadIdx.x; c0 < nch; c0 += 4 * 256) {
      u32x4 v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = src[min(c0 + 256 * r, nch - 1)];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (c0 + 256 * r < nch) dst[c0 + 256 * r] = v[r];
    }
  }
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, hipStream_t st) {
  if (a.lc_first < 0 || a.lc_count < 1 || a.lc_first + a.lc_count > a.layer_count) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_kernel, dim3(a.B * a.Hkv * a.nsplit, a.lc_count), dim3(256), 0, st, a);
  return hipGetLastError();
}

int gather_share() { return kShare; }

}  // namespace sekv
