// Internal definitions shared by the SeKV HIP kernels and the host runtime:
// storage layouts in HBM, per-sequence metadata, kernel argument blocks and
// launcher declarations.  Not part of the public ABI (include/sekv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sekv {

typedef uint16_t bf16_t;

// ---------------------------------------------------------------------------
// Storage layouts.  Every matrix the decode kernel streams is stored in the
// lane order of the MFMA operand that consumes it, so that one wave-wide
// 16-byte (or 8-byte) load per lane reads 1 KB (512 B) of contiguous HBM.
//
// MFMA operand conventions used throughout (gfx950, wave64):
//   v_mfma_f32_16x16x32_bf16  A[i][k]: lane = i + 16*(k/8), element k%8
//                             B[k][j]: lane = j + 16*(k/8), element k%8
//   v_mfma_f32_16x16x16_bf16  A[i][k]: lane = i + 16*(k/4), element k%4
//                             B[k][j]: lane = j + 16*(k/4), element k%4
//   both                      D[i][j]: lane = j + 16*(i/4), element i%4
// ---------------------------------------------------------------------------

// Row-major "K rows" (resident keys, and V^K^T of a span): A operand of
// 16x16x32 with i = row within a 16-row block and k = dim within a 32-dim
// slice.  Tiles ordered [row/16][dim/32][lane][8].
__host__ __device__ inline int64_t krow_off(int64_t row, int dim, int D) {
  const int i = (int)(row & 15), s = dim >> 5;
  const int lane = i + 16 * ((dim & 31) >> 3), e = dim & 7;
  return (row >> 4) * 16 * D + s * 512 + lane * 8 + e;
}

// Resident values: A operand of 16x16x32 computing O^T[dim][head] =
// V^T[dim][rows] P[rows][head] over 32-row blocks.  k = 8*(lane/16) + e maps
// to row 4*(lane/16) + e (e < 4) or 16 + 4*(lane/16) + e - 4 (e >= 4) of the
// block, which is the row order in which the score MFMA leaves P in its
// D operand.  Tiles ordered [row/32][dim/16][lane][8].
__host__ __device__ inline int64_t vrow_off(int64_t row, int dim, int D) {
  const int rr = (int)(row & 31), half = rr >> 4, rq = rr & 15;
  const int lane = (dim & 15) + 16 * (rq >> 2), e = 4 * half + (rq & 3);
  return (row >> 5) * 32 * D + (dim >> 4) * 512 + lane * 8 + e;
}

// A operand of 16x16x16 for a matrix with Kd columns (multiple of 16):
// tiles ordered [i/16][k/16][lane][4].
__host__ __device__ inline int64_t a16_off(int64_t i, int k, int Kd) {
  const int lane = (int)(i & 15) + 16 * ((k & 15) >> 2), e = k & 3;
  return ((i >> 4) * (Kd >> 4) + (k >> 4)) * 256 + lane * 4 + e;
}

// One span's factor blob (per layer and KV head), with rk key and rv value
// components stored (multiples of 16, the MFMA tile; see BlobRef), n_pad = n
// rounded up to 16:
//   VKt  [rk][d]   right key factors V^K^T       krow_off(i, dim, d)
//   VV   [d][rv]   right value factors V^V       a16_off(dim, i, rv)
//   smK  [rk] fp32 sigma^K * m^K
//   smV  [rv] fp32 sigma^V * m^V
//   UK   [n_pad][rk] left key factors U^K        a16_off(t, i, rk)
//   UVt  [rv][n_pad] left value factors U^V^T    a16_off(i, t, n_pad)
// Rows/cols past n and components past the kept ones are zero.  Blobs start
// on 256-byte boundaries.
struct Blob {
  static __host__ __device__ inline int npad(int n) { return (n + 15) & ~15; }
  static __host__ __device__ inline int64_t off_vkt() { return 0; }
  static __host__ __device__ inline int64_t off_vv(int rk, int D) { return 2LL * rk * D; }
  static __host__ __device__ inline int64_t off_smk(int rk, int rv, int D) { return 2LL * (rk + rv) * D; }
  static __host__ __device__ inline int64_t off_smv(int rk, int rv, int D) { return off_smk(rk, rv, D) + 4LL * rk; }
  static __host__ __device__ inline int64_t off_uk(int rk, int rv, int D) { return off_smv(rk, rv, D) + 4LL * rv; }
  static __host__ __device__ inline int64_t off_uvt(int rk, int rv, int D, int n) {
    return off_uk(rk, rv, D) + 2LL * npad(n) * rk;
  }
  static __host__ __device__ inline int64_t bytes(int rk, int rv, int D, int n) {
    return (off_uvt(rk, rv, D, n) + 2LL * npad(n) * rv + 255) & ~255LL;
  }
};

// Where the blob of (layer l, KV head g, span) sits and what it holds: a
// uint2 {x: byte offset / 256 within layer l's factor region, y: rk | rv << 16}.
// Table [L][Hkv][total spans]; the layer's region starts at layer_off[l].
__host__ __device__ inline int bref_rk(uint2 r) { return (int)(r.y & 0xffffu); }
__host__ __device__ inline int bref_rv(uint2 r) { return (int)(r.y >> 16); }

// Stored rank of a span's K or V factorization that keeps `kept` components:
// rounded up to the 16-wide MFMA tile, at least one tile.
__host__ __device__ inline int stored_rank(int kept) { return kept <= 16 ? 16 : (kept + 15) & ~15; }
// Component gate test: kept iff eps <= 0 or m >= eps (NaN gates fail it).
__host__ __device__ inline bool gate_kept(float m, float eps) { return eps <= 0.f || m >= eps; }

// Per-sequence metadata (device copy used by every kernel).
// Summary keys s of one (b, l, h): s_pad span slots x d4 = d' rounded up to 4
// dims (zeros past d'), in blocks of 64 spans x 4 dims: lane S % 64 of a
// routing wave reads its span's 4 dims as one 16-byte load, and the wave's
// 64 loads are 1 KB contiguous.
__host__ __device__ inline int dp_pad4(int dp) { return (dp + 3) & ~3; }
__host__ __device__ inline int64_t skey_index(int S, int j, int d4) {
  return ((int64_t)(S >> 6) * (d4 >> 2) + (j >> 2)) * 256 + (S & 63) * 4 + (j & 3);
}

struct BMeta {
  int32_t n_spans;      // N_S(b)
  int32_t n_raw;        // N_raw(b)
  int32_t n_res;        // N_raw + N_S
  int32_t n_res_pad;    // n_res rounded up to 64
  int32_t s_pad;        // N_S rounded up to 64 (span slots of one (l, h) of s)
  int32_t pad_;
  int64_t span_base;    // first span of b in the span tables
  int64_t raw_base;     // first raw token of b in raw_pos
  int64_t tok_base;     // first token of b's spans in the concatenated U order
  int64_t res_base;     // element offset of (b, l=0, g=0) in K/V resident rows
  int64_t s_base;       // element offset of (b, l=0, h=0) in s
};

// Routed spans one work item may take (one per lane of a wave).
constexpr int kMaxSpanList = 64;
// Mask words per (b, l, h) the decode kernel handles (65536 spans).
constexpr int kMaxWords = 1024;

// Decode work: one workgroup of 4 waves per item.  Item j of the nj items of
// a KV head (b, g) takes the resident 32-row steps [step_begin, step_end) and
// the j-th of nj equal shares of the union of the routed spans of (b, l, g);
// it writes its softmax partial to `slot` (the slots of one (b, g) are
// contiguous).
struct WorkItem {
  int32_t b, g;
  int32_t j, nj;                    // union share j of nj of (b, g)
  int32_t step_begin, step_end;     // resident 32-row steps of (b, g)
  int32_t slot;                     // partial slot
  int32_t pad;
};

struct AttendArgs {
  const bf16_t* q;          // [B][Lc][Hq][D]
  const uint64_t* mask;     // [B][Lc][Hq][W]
  const BMeta* meta;
  const WorkItem* items;
  const bf16_t* kres;
  const bf16_t* vres;
  const float* logn;        // [span] ln n_S
  const int32_t* span_len;  // [span]
  const uint2* bref;        // [L][Hkv][total_spans] blob references
  const int64_t* layer_off; // [L + 1] byte offset of each layer's factor region
  const uint8_t* pool;      // factor pool (HBM tier) or staging ring (pinned
                            // tier: the call's layers, blobs at their pool offsets)
  float* part;              // [Lc][n_items][G][D + 2] softmax partials
  int64_t total_spans;
  int32_t pool_layer0;      // layer whose region starts `pool` (0; a ring slot: its layer)
  int32_t layer_begin, layer_count, n_items;
  int32_t lc_first, lc_count;   // this launch: layers [lc_first, lc_first + lc_count) of the call
  int32_t B, L, Hq, Hkv, W, max_spans;
  float scale;              // 1/sqrt(d)
  int32_t stream;           // 1: the streamed operands (resident rows, factor
                            // blobs) are loaded with the non-temporal hint
                            // (chooses the kernel instance on the host)
};

struct MergeArgs {
  const float* part;
  const WorkItem* items;
  const int32_t* bg_first;  // [B*Hkv][2]: first partial slot of (b, g), slot count
  float* out;               // [B][Lc][Hq][D]
  int32_t layer_count, n_items, B, Hq, Hkv;
};

struct RouteArgs {
  const bf16_t* q;          // [B][Lc][Hq][D]
  const float* tau;         // [Lc][Hq]
  const float* W;           // [L][Hq][dp][D]
  const float* s;
  const BMeta* meta;
  uint64_t* mask;           // [B][Lc][Hq][Wd]
  float* alpha;             // [B][Lc][Hq][Wd*64] sigmoid of the score, or NULL
  float* score;             // [B][Lc][Hq][Wd*64] score a = u . s (library
                            // scratch the budget kernels rank), or NULL
  uint32_t* packed;         // [B][Lc][Hq][Wd][64] order keys of the routed
                            // spans of each mask word, packed at the start of
                            // the word's 64 slots in span order (scratch of
                            // the pooled budget), or NULL
  int32_t layer_begin, layer_count;
  int32_t B, L, Hq, Hkv, D, dp, Wd, cap;
  int32_t budget;           // pooled budget per sequence (route_pool_kernel)
  int32_t stream;           // 1: the summary keys are loaded with the
                            // non-temporal hint (chooses the kernel instance)
};

struct CalibArgs {
  const float* alpha;       // [B][Lc][Hq][Wd*64]
  const BMeta* meta;
  float* tau_out;           // [Lc][Hq]
  int32_t layer_count, B, Hq, Wd;
  float frac;
};

// Pinned-tier gather (see gather.hip): the union's blobs copied from the
// mapped pinned pool to the same layer-relative offsets of the HBM ring.
struct GatherArgs {
  const uint64_t* mask;      // [B][Lc][Hq][W]
  const BMeta* meta;
  const int32_t* span_len;
  const uint2* bref;         // [L][Hkv][total_spans] blob references
  const int64_t* layer_off;  // [L + 1]
  const uint8_t* host_pool;  // device address of the mapped pinned factor pool
  uint8_t* ring;             // HBM staging ring (slot): layer l at layer_off[l] - layer_off[ring_layer0]
  int2* stat;                // [Lc][B][Hkv]: union spans, union blob bytes / 256 (or NULL)
  int64_t total_spans;
  int32_t layer_begin, layer_count, B, Hq, Hkv, W, G, D, nsplit;
  int32_t lc_first, lc_count;   // this launch: layers [lc_first, lc_first + lc_count) of the call
  int32_t ring_layer0;      // layer whose region starts `ring`
};

// ------------------------------------------------------------ launchers ---
// With ev_start / ev_stop the launch records them in its dispatch packet
// (hipExtLaunchKernel): their interval is the kernel's own execution.
hipError_t launch_attend(const AttendArgs& a, int D, int G, int R, hipStream_t st,
                         hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_merge(const MergeArgs& a, int D, int G, hipStream_t st);
hipError_t launch_route(const RouteArgs& a, hipStream_t st);
hipError_t launch_route_cap(const RouteArgs& a, hipStream_t st);
hipError_t launch_route_pool(const RouteArgs& a, hipStream_t st);
hipError_t launch_calibrate(const CalibArgs& a, hipStream_t st);
bool attend_supported(int D, int G, int R);
// Workgroups of the attention kernel for (D, G, R) with W mask words that the
// device can hold resident at once (CUs x workgroups per CU).
hipError_t attend_slots(int D, int G, int R, int W, int device, int* slots);

struct SplitArgs {
  const float* H;           // [B][T]
  int32_t* span_start;      // [B][S_max]
  int32_t* span_len;        // [B][S_max]
  int32_t* raw_pos;         // [B][T]
  int32_t* counts;          // [B][2] (N_S, N_raw)
  int32_t* scratch;         // [B][2][T/2 + 2]
  int32_t B, T, S_max, l_min;
  double alpha_sp;
};
hipError_t launch_span_split(const SplitArgs& a, hipStream_t st);

// Stored ranks of every span's K and V factorization (span split scratch
// layout): ranks[((b L + l) Hkv + g) S_max + S] = rk | rv << 16.
struct RankArgs {
  const float* gates;       // [B][L][Hkv][2][S_max][R] or NULL (m = 1)
  const int32_t* span_len;  // [B][S_max]
  const int32_t* counts;    // [B][2] (N_S, N_raw)
  uint32_t* ranks;          // [B][L][Hkv][S_max]
  int32_t B, L, Hkv, R, S_max;
  float gate_eps;
};
hipError_t launch_ranks(const RankArgs& a, hipStream_t st);

struct PackArgs {
  const bf16_t* K;          // [B][L][Hkv][T][D]
  const bf16_t* V;
  const float* H;           // [B][T]
  const float* W;           // [L][Hq][dp][D]
  const float* gates;       // [B][L][Hkv][2][S_max][R] or NULL
  const BMeta* meta;
  const int32_t* span_start;  // concatenated over b
  const int32_t* span_len;
  const int32_t* raw_pos;
  const uint2* bref;        // [L][Hkv][total_spans] blob references
  bf16_t* kres;
  bf16_t* vres;
  float* s;
  uint8_t* pool;            // device factor destination: one layer's region
                            // (pool + layer_off[layer], or a staging buffer)
  int64_t total_spans;
  float gate_eps;           // components with gate < gate_eps are dropped (if > 0)
  int32_t B, L, Hq, Hkv, D, T, R, dp, S_max;
  int32_t layer;            // layer for the per-layer SVD launch
  int32_t max_raw, max_spans;
  int32_t oversample, power_iters;
  uint64_t seed;
  // batched mode (sekv_rsvd_batched): matrices given directly, fp32 outputs
  const bf16_t* A;
  const int64_t* mat_row_off;
  const int32_t* mat_rows;
  float* out_U;             // [count][max_rows][R]
  float* out_S;             // [count][R]
  float* out_Vt;            // [count][R][D]
  int32_t count, max_rows;
};
hipError_t launch_pack_raw(const PackArgs& a, hipStream_t st);
hipError_t launch_summaries(const PackArgs& a, hipStream_t st);
hipError_t launch_rsvd(const PackArgs& a, hipStream_t st);
hipError_t launch_rsvd_batched(const PackArgs& a, hipStream_t st);
hipError_t launch_gather(const GatherArgs& a, hipStream_t st);
int gather_share();   // union spans per gather workgroup

}  // namespace sekv
