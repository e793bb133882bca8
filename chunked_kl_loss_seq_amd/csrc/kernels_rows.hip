// Per-token kernels of the fused chunked KL loss: valid-token count, the row
// pass over a chunk (log-normaliser, teacher softmax over the cached top-K,
// gather, KL, in-place logit gradient and top-K scatter) and the final loss
// reduction.
//
// Definitions followed (the pages print no formulas; these are the plain
// readings that the rest of the pages support):
//  * teacher distribution = softmax over the K cached teacher logits only
//    ("A New Trick Slashes the Cost of Shrinking Giant AI Models", section
//    "What did the researchers change?"; "Making Knowledge Distillation Cheap
//    Enough to Run at Scale" (elseif.net), limitations paragraph);
//  * student log-probabilities = full-vocabulary log-softmax, the vocabulary x
//    sequence grid of section "Why is this so hard to do cheaply?";
//  * loss = mean over valid positions of KL(p_T || p_S); its logit gradient is
//    w_r (softmax(z_r) - scatter(p_T,r)) with w_r = mask_r / n_valid.
//
// Chunk workspace.  The logits GEMM leaves, per token r and 128-id slice s,
// the slice max m_rs and the sum of exp(z - m_rs) (the "slice pairs"), and per
// logit the value p = exp(z - m_rs) in the element type T of the gradient,
// laid out in 64 x 64 tiles (tile_off below).  Then, for each chunk:
//  0. id tables (before the logits GEMM): per row and slice, a 128-bit mask of
//     the cached ids and the count of cached ids below the slice; per cached id
//     its rank among the row's distinct ids.  The logits GEMM copies the fp32
//     logit at each masked position out of its accumulators, before they
//     become exp values, to zs[r][rank]: the exact logit at each cached id;
//  1. row_stats: lse_r = merge of the slice pairs; teacher softmax; the cached
//     ids' logits z from zs; KL_r; the per-slice gradient factor
//     f_rs = w_r exp(m_rs - lse_r) (written over the pair's sum); and the exact
//     gradient value at each cached id, w_r (exp(z - lse_r) - p_T);
//  2. dense: G = f_rs p over every tile, in place (same element, same type);
//  3. scatter: G at the cached ids <- the exact values of step 1.
// With a mask, each chunk is first compacted: its valid rows (H, cached ids
// and logits) are gathered, in order, to the front of chunk buffers, and every
// kernel of the chunk runs on those `live` rows only.  Masked rows get no
// logits and no GEMM work; they report KL 0 and log-normaliser 0, and their
// dH rows are written as zeros.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>

#include "launch.hpp"

namespace ckl {

namespace {

constexpr int kRowThreads = 256;
constexpr int kKPT = kMaxK / kRowThreads;  // cached ids per thread

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Scalars {
  long long n_valid;
  float scale;
  float pad;
  unsigned err;  // at kErrOffset: flags of launch_id_tables, cleared by the valid count
};
static_assert(offsetof(Scalars, err) == kErrOffset, "error flags offset");
static_assert(offsetof(Scalars, scale) == kScaleOffset, "gradient weight offset");

// Element (row r, column v) of a 64 x 64-tiled matrix whose tile rows are
// `blk` elements apart.
__device__ inline int64_t tile_off(int64_t r, int64_t v, int64_t blk) {
  return (r >> 6) * blk + (v >> 6) * 4096 + (r & 63) * 64 + (v & 63);
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// (m, s) summarises a set of logits as max m and sum of exp(z - m).
__device__ inline void lse_merge(float& m, float& s, float m2, float s2) {
  if (s2 == 0.f) return;
  if (s == 0.f) {
    m = m2;
    s = s2;
    return;
  }
  const float M = fmaxf(m, m2);
  s = s * __expf(m - M) + s2 * __expf(m2 - M);
  m = M;
}

template <int NT>
__device__ inline float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

template <int NT>
__device__ inline float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r += red[i];
  return r;
}

template <int NT>
__device__ inline void block_lse_merge(float& m, float& s, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    lse_merge(m, s, m2, s2);
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[2 * w] = m;
    red[2 * w + 1] = s;
  }
  __syncthreads();
  m = red[0];
  s = red[1];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) lse_merge(m, s, red[2 * i], red[2 * i + 1]);
}

template <typename T>
__device__ inline float to_f(T x) {
  return (float)x;
}

// ------------------------------------------------------------------ valid count
__global__ void __launch_bounds__(1024) mask_count_kernel(const uint8_t* __restrict__ mask, int64_t N,
                                                         Scalars* __restrict__ out) {
  __shared__ long long red[16];
  long long c = 0;
  if (mask) {
    for (int64_t i = threadIdx.x; i < N; i += 1024) c += mask[i] != 0;
  } else {
    c = threadIdx.x == 0 ? N : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long t = 0;
    for (int i = 0; i < 16; ++i) t += red[i];
    out->n_valid = t;
    out->scale = t > 0 ? (float)(1.0 / (double)t) : 0.f;
    out->pad = 0.f;
    out->err = 0u;
  }
}

// Compaction of one chunk of `rows` positions (mask, row outputs and the
// index arrays relative to the chunk): vidx[i] = the chunk row of the i-th
// valid position, pos[j] = the compact index of chunk row j or -1, *live =
// the valid count.  Masked rows' KL and log-normaliser are written as 0 here.
// One workgroup; thread t takes a contiguous run of rows.
__global__ void __launch_bounds__(1024) compact_scan_kernel(const uint8_t* __restrict__ mask, int64_t rows,
                                                           int* __restrict__ vidx, int* __restrict__ pos,
                                                           int* __restrict__ live, float* __restrict__ kl_out,
                                                           float* __restrict__ lse_out) {
  __shared__ int red[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t per = (rows + 1023) / 1024;
  const int64_t j0 = min(rows, tid * per), j1 = min(rows, j0 + per);
  int n = 0;
  for (int64_t j = j0; j < j1; ++j) n += mask[j] != 0;
  // exclusive prefix of n over threads: within the wave, then over waves
  int x = n;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[w] = x;
  __syncthreads();
  int before = x - n;
  for (int i = 0; i < w; ++i) before += red[i];
  for (int64_t j = j0; j < j1; ++j) {
    if (mask[j] != 0) {
      vidx[before] = (int)j;
      pos[j] = before++;
    } else {
      pos[j] = -1;
      kl_out[j] = 0.f;
      if (lse_out) lse_out[j] = 0.f;
    }
  }
  if (tid == 1023) *live = before;
}

// Gather of the live rows: Hc[i] = H[vidx[i]], ids and teacher logits alike,
// for i < *live; rows [*live, next multiple of 256) of Hc are zeroed, since
// the logits and dW contractions read whole 256-row tiles and 64-row k-steps
// (their gradient rows are zero, and zero times a stale NaN would not be).
// One workgroup per row; d % 8 == 0.
template <typename T>
__global__ void __launch_bounds__(256) compact_gather_kernel(const int* __restrict__ vidx, const int* __restrict__ live,
                                                            int64_t rows_alloc, const T* __restrict__ H, int64_t d,
                                                            const int32_t* __restrict__ ids,
                                                            const float* __restrict__ tlogit, int K,
                                                            T* __restrict__ Hc, int32_t* __restrict__ ids_c,
                                                            float* __restrict__ tl_c) {
  const int64_t i = blockIdx.x;
  const int n = *live;
  const int64_t zero_end = min(rows_alloc, ((int64_t)n + 255) / 256 * 256);
  if (i >= zero_end) return;
  constexpr int EPC = 16 / (int)sizeof(T);
  T* dst = Hc + i * d;
  if (i < n) {
    const int64_t src = vidx[i];
    const T* s = H + src * d;
    for (int64_t c = threadIdx.x; c < d / EPC; c += 256) ((u32x4*)dst)[c] = ((const u32x4*)s)[c];
    for (int k = threadIdx.x; k < K; k += 256) {
      ids_c[i * K + k] = ids[src * K + k];
      tl_c[i * K + k] = tlogit[src * K + k];
    }
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t c = threadIdx.x; c < d / EPC; c += 256) ((u32x4*)dst)[c] = z;
  }
}

// ------------------------------------------------------------------ 0. id tables
// Tables of the cached ids of chunk rows, in the layout the logits GEMM reads
// (pair = two consecutive 128-id slices = one 256-id tile of the vocabulary;
// rows padded to cpad, a multiple of 256):
//   bits[pair][row][2]  128-bit mask of the row's cached ids in each slice
//   pre[pair][row]      two uint16: the number of the row's distinct cached
//                       ids below each of the pair's two slices (below 128 s
//                       for a slice s past the vocabulary: the row's total)
//   rank[row][k]        pre of id k's slice + the mask bits below id k: the
//                       place of id k's logit in zs, or -1 for an id outside
//                       [0, V)
// One workgroup of four waves takes four consecutive rows (wave w: row
// 4 b + w), so that the four rows' entries of a pair, adjacent in memory, go
// out as whole 128-byte lines.  The masks of up to kTabSlices slices at a time
// are built with LDS atomics; an id whose bit is already set is a repeat.
// Rows at and past *live (compacted chunk) and past `rows` get empty tables.
// Flags: 1 = id outside [0, V), 2 = repeated id.
constexpr int kTabSlices = 1024;
constexpr int kIdsPerLane = kMaxK / 64;

__global__ void __launch_bounds__(256) id_table_kernel(const int32_t* __restrict__ ids, int K, int64_t V, int n_slices,
                                                      int64_t cpad, int64_t rows, const int* __restrict__ live,
                                                      u32x4* __restrict__ bits, uint32_t* __restrict__ pre,
                                                      int32_t* __restrict__ rank, unsigned* __restrict__ err) {
  __shared__ u32x4 mb[4][kTabSlices + 4];  // rows 64 bytes of banks apart
  __shared__ int sp[4][kTabSlices + 1];
  const int64_t r0 = (int64_t)blockIdx.x * 4;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t r = r0 + wv;
  const bool row_in = r < rows;
  const bool row_live = row_in && (live == nullptr || r < *live);
  const int nq = (K + 63) / 64;  // ids per lane in use (uniform)
  int iv[kIdsPerLane], rk[kIdsPerLane];
  unsigned flags = 0;
#pragma unroll
  for (int q = 0; q < kIdsPerLane; ++q) {
    if (q >= nq) break;
    const int k = lane + 64 * q;
    iv[q] = -1;
    rk[q] = -1;
    if (row_live && k < K) {
      const int id = ids[r * K + k];
      if (id >= 0 && id < V)
        iv[q] = id;
      else
        flags |= 1u;
    }
  }
  int carry = 0;  // this wave's row: distinct ids in the slices before the pass
  for (int base = 0; base < n_slices; base += kTabSlices) {
    const int np = min(kTabSlices, n_slices - base);
    for (int i = tid; i < 4 * kTabSlices; i += 256) mb[i / kTabSlices][i % kTabSlices] = u32x4{0u, 0u, 0u, 0u};
    // (the 4 padding entries of each row are never read)
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kIdsPerLane; ++q) {
      if (q >= nq) break;
      const int id = iv[q];
      const int s = (id >> 7) - base;
      if (id >= 0 && s >= 0 && s < np) {
        const unsigned bit = 1u << (id & 31);
        const unsigned old = atomicOr(&((unsigned*)&mb[wv][s])[(id >> 5) & 3], bit);
        if (old & bit) flags |= 2u;
      }
    }
    __syncthreads();
    // exclusive prefix of the row's per-slice counts: lane l takes slices
    // 8 l .. 8 l + 7 of the pass, then a wave scan of the lane totals
    int cnt[kTabSlices / 64];
    int local = 0;
#pragma unroll
    for (int i = 0; i < kTabSlices / 64; ++i) {
      const int s = lane * (kTabSlices / 64) + i;
      cnt[i] = 0;
      if (s < np) {
        const u32x4 w = mb[wv][s];
        cnt[i] = __builtin_popcount(w.x) + __builtin_popcount(w.y) + __builtin_popcount(w.z) + __builtin_popcount(w.w);
      }
      local += cnt[i];
    }
    int x = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    const int total = __shfl(x, 63);
    int run = carry + x - local;
#pragma unroll
    for (int i = 0; i < kTabSlices / 64; ++i) {
      const int s = lane * (kTabSlices / 64) + i;
      if (s < np) sp[wv][s] = run;
      run += cnt[i];
    }
    if (lane == 0) sp[wv][np] = carry + total;  // a slice past the pass (or the vocabulary)
    __syncthreads();
    // the pass's pairs: the masks of one pair and the four rows are one
    // 128-byte line, written by 8 consecutive lanes (row i, slice half h);
    // the count pairs of the four rows are 16 bytes, one lane per pair
    const int npairs = (np + 1) / 2;
    for (int e = tid; e < 8 * npairs; e += 256) {
      const int pl = e >> 3, i = (e >> 1) & 3, h = e & 1;
      const int sl = 2 * pl + h;
      bits[((base / 2 + pl) * cpad + r0 + i) * 2 + h] = sl < np ? mb[i][sl] : u32x4{0u, 0u, 0u, 0u};
    }
    for (int pl = tid; pl < npairs; pl += 256) {
      const int64_t pr = base / 2 + pl;
      uint32_t pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sl = 2 * pl;
        pv[i] = (uint32_t)sp[i][sl] | ((uint32_t)sp[i][sl + 1 < np ? sl + 1 : np] << 16);
      }
      *(u32x4*)(pre + pr * cpad + r0) = u32x4{pv[0], pv[1], pv[2], pv[3]};
    }
#pragma unroll
    for (int q = 0; q < kIdsPerLane; ++q) {
      if (q >= nq) break;
      const int id = iv[q];
      const int s = (id >> 7) - base;
      if (id >= 0 && s >= 0 && s < np) {
        const u32x4 w = mb[wv][s];
        const int wi = (id >> 5) & 3;
        const unsigned below = (1u << (id & 31)) - 1u;
        int c = sp[wv][s] + __builtin_popcount(w[wi] & below);
        if (wi > 0) c += __builtin_popcount(w.x);
        if (wi > 1) c += __builtin_popcount(w.y);
        if (wi > 2) c += __builtin_popcount(w.z);
        rk[q] = c;
      }
    }
    carry += total;
    __syncthreads();
  }
  if (row_in) {
#pragma unroll
    for (int q = 0; q < kIdsPerLane; ++q) {
      if (q >= nq) break;
      const int k = lane + 64 * q;
      if (k < K) rank[r * K + k] = rk[q];
    }
  }
  if (err != nullptr) {
    const unsigned long long any = __ballot(flags != 0);
    if (any != 0ull) {
      unsigned f = flags;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o);
      if (lane == 0) atomicOr(err, f);
    }
  }
}

// ------------------------------------------------------------------ 1. row statistics
// One workgroup per token row.
template <typename T>
__global__ void __launch_bounds__(kRowThreads) row_stats_kernel(RowArgs a) {
  constexpr int NT = kRowThreads;
  __shared__ float red[2 * (NT / 64)];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  if (a.live != nullptr && r >= *a.live) return;  // past the compacted rows
  // row outputs (and a saved log-normaliser) belong to the chunk row this
  // compacted row came from
  const int64_t ro = a.vidx != nullptr ? a.vidx[r] : r;
  const Scalars* sc = (const Scalars*)a.scal;
  const float scale = sc ? sc->scale : a.scale_value;
  const bool valid = a.mask == nullptr || a.mask[r] != 0;
  const float w = valid ? (a.gscale ? scale * *a.gscale : scale) : 0.f;
  float2* prow = a.part + r * a.n_slices;

  // student log-normaliser: merged from the slice pairs, or the value a
  // forward pass over the same inputs saved (bitwise the same: the logits
  // GEMM and the merge order do not depend on the chunking)
  float lse;
  if (a.lse_in) {
    lse = a.lse_in[ro];
  } else {
    float m = -INFINITY, s = 0.f;
    for (int p = tid; p < a.n_slices; p += NT) {
      const float2 q = prow[p];
      lse_merge(m, s, q.x, q.y);
    }
    block_lse_merge<NT>(m, s, red);
    lse = m + logf(s);
  }

  // teacher softmax over the cached logits; gather; KL; exact values at the ids
  const int K = a.K;
  float tv[kKPT];
  int iv[kKPT];
  float tmax = -INFINITY;
#pragma unroll
  for (int q = 0; q < kKPT; ++q) {
    const int k = tid + q * NT;
    tv[q] = -INFINITY;
    iv[q] = 0;
    if (k < K) {
      tv[q] = a.tlogit[r * K + k];
      iv[q] = a.ids[r * K + k];
      tmax = fmaxf(tmax, tv[q]);
    }
  }
  const float tau = block_max<NT>(tmax, red);
  float se = 0.f;
#pragma unroll
  for (int q = 0; q < kKPT; ++q)
    if (tid + q * NT < K) se += __expf(tv[q] - tau);
  const float lse_t = tau + logf(block_sum<NT>(se, red));
  float klp = 0.f;
#pragma unroll
  for (int q = 0; q < kKPT; ++q) {
    const int k = tid + q * NT;
    if (k < K) {
      const int id = iv[q];
      // the fp32 logit the contraction computed at this id (an id outside
      // [0, V) has no rank: it is flagged and left out)
      const int rk = a.rank[r * K + k];
      const float zg = rk >= 0 ? a.zs[r * K + rk] : 0.f;
      const float lpt = tv[q] - lse_t;
      const float pt = __expf(lpt);
      if (rk >= 0) klp += pt * (lpt - (zg - lse));
      a.scat[r * K + k] = (valid && rk >= 0) ? w * __expf(zg - lse) - w * pt : 0.f;
      if (a.zg_dbg) {
        a.zg_dbg[r * K + k] = zg;
        a.sid_dbg[r * K + k] = id;
      }
    }
  }
  const float kl = block_sum<NT>(klp, red);

  // every thread has read the pairs it needs; now the factors replace the sums
  __syncthreads();
  for (int p = tid; p < a.n_slices; p += NT) {
    const float2 q = prow[p];
    prow[p].y = valid ? w * __expf(q.x - lse) : 0.f;
  }
  if (tid == 0) {
    if (a.kl_out) a.kl_out[ro] = valid ? kl : 0.f;
    if (a.lse_out) a.lse_out[ro] = valid ? lse : 0.f;
  }
}

// ------------------------------------------------------------------ 2. dense gradient
// One workgroup per 64 x 64 tile: thread t owns row t / 4, columns
// 16 (t % 4) .. + 15.  G = f p in place; zero for ids >= V and rows >= rows.
template <typename T>
__global__ void __launch_bounds__(256) dense_kernel(RowArgs a) {
  const int64_t tb = blockIdx.y, vb = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t r = tb * 64 + (tid >> 2);
  const int64_t v0 = vb * 64 + (tid & 3) * 16;
  T* g = (T*)a.P + tile_off(r, v0, a.pblk);
  // rows past the chunk, or past its compacted rows, hold no exp values
  // (possibly not even numbers): they are written as zeros without being read
  // into the product
  const bool row_ok = r < a.rows && (a.live == nullptr || r < *a.live);
  float f = 0.f;
  if (row_ok && v0 < a.V) f = a.part[r * a.n_slices + (v0 >> 7)].y;
  if constexpr (sizeof(T) == 2) {
    typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 x = *(const bf16x8*)(g + 8 * h);
      bf16x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (__bf16)((row_ok && v0 + 8 * h + e < a.V) ? f * (float)x[e] : 0.f);
      *(bf16x8*)(g + 8 * h) = y;
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      f32x4 x = *(const f32x4*)(g + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (row_ok && v0 + 4 * h + e < a.V) ? f * x[e] : 0.f;
      *(f32x4*)(g + 4 * h) = x;
    }
  }
}

// ------------------------------------------------------------------ 3. top-K scatter
template <typename T>
__global__ void __launch_bounds__(256) scatter_kernel(RowArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.rows * a.K) return;
  const int64_t r = i / a.K;
  if (a.mask != nullptr && a.mask[r] == 0) return;
  if (a.live != nullptr && r >= *a.live) return;  // past the compacted rows: no ids
  const int id = a.ids[i];
  if (id < 0 || id >= a.V) return;  // flagged by the id tables; nothing is written
  ((T*)a.P)[tile_off(r, id, a.pblk)] = (T)a.scat[i];
}

// ------------------------------------------------------------------ debug helpers
// Slice pairs and exp values of caller-given fp32 logits (the same quantities
// the logits GEMM leaves), one workgroup per (128-id slice, row).
template <typename T>
__global__ void __launch_bounds__(128) partials_from_z_kernel(const float* __restrict__ Z, int64_t ldz, int64_t V,
                                                              float2* __restrict__ part, int n_slices, T* P,
                                                              int64_t pblk) {
  __shared__ float red[4];
  const int64_t r = blockIdx.y;
  const int slice = blockIdx.x;
  const int64_t j = (int64_t)slice * 128 + threadIdx.x;
  const bool ok = j < V;
  const float z = ok ? Z[r * ldz + j] : -INFINITY;
  float m = wave_max(z);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(red[0], red[1]);
  __syncthreads();
  const float e = ok ? __expf(z - m) : 0.f;
  if (ok) P[tile_off(r, j, pblk)] = (T)e;
  float s = wave_sum(e);
  if ((threadIdx.x & 63) == 0) red[2 + (threadIdx.x >> 6)] = s;
  __syncthreads();
  if (threadIdx.x == 0) part[r * n_slices + slice] = make_float2(m, red[2] + red[3]);
}

__global__ void __launch_bounds__(256) zs_from_z_kernel(const float* __restrict__ Z, int64_t ldz,
                                                        const int32_t* __restrict__ ids,
                                                        const int32_t* __restrict__ rank, int64_t rows, int K,
                                                        float* __restrict__ zs) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * K) return;
  const int64_t r = i / K;
  const int rk = rank[i];
  if (rk >= 0) zs[r * K + rk] = Z[r * ldz + ids[i]];
}

template <typename T>
__global__ void __launch_bounds__(256) untile_kernel(const T* __restrict__ P, int64_t pblk, int64_t R, int64_t V,
                                                     T* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= R * V) return;
  const int64_t r = i / V, v = i - r * V;
  out[i] = P[tile_off(r, v, pblk)];
}

// ------------------------------------------------------------------ finalize
__global__ void __launch_bounds__(1024) finalize_kernel(const float* __restrict__ kl, int64_t N,
                                                       const Scalars* __restrict__ sc, float* __restrict__ out) {
  __shared__ double red[16];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < N; i += 1024) acc += (double)kl[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < 16; ++i) t += red[i];
    const long long n = sc->n_valid;
    *out = n > 0 ? (float)(t / (double)n) : 0.f;
  }
}

}  // namespace

hipError_t launch_compact(Dtype dt, const uint8_t* mask, int64_t rows, int64_t rows_alloc, const void* H,
                          int64_t d, const int32_t* ids, const float* tlogit, int K, int* vidx, int* pos,
                          int* live, float* kl_out, float* lse_out, void* Hc, int32_t* ids_c, float* tl_c,
                          hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(1024), 0, s, mask, rows, vidx, pos, live, kl_out, lse_out);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(compact_gather_kernel<__bf16>, dim3((unsigned)rows_alloc), dim3(256), 0, s, vidx, live,
                       rows_alloc, (const __bf16*)H, d, ids, tlogit, K, (__bf16*)Hc, ids_c, tl_c);
  else
    hipLaunchKernelGGL(compact_gather_kernel<float>, dim3((unsigned)rows_alloc), dim3(256), 0, s, vidx, live,
                       rows_alloc, (const float*)H, d, ids, tlogit, K, (float*)Hc, ids_c, tl_c);
  return hipGetLastError();
}

hipError_t launch_id_tables(const int32_t* ids, int K, int64_t rows, int64_t V, const int* live, void* bits,
                            void* pre, int64_t cpad, int32_t* rank, unsigned* err, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (cpad % 256 != 0 || cpad < rows) return hipErrorInvalidValue;
  const int n_slices = (int)((V + 127) / 128);
  hipLaunchKernelGGL(id_table_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, ids, K, V, n_slices, cpad,
                     rows, live, (u32x4*)bits, (uint32_t*)pre, rank, err);
  return hipGetLastError();
}

hipError_t launch_zs_from_z(const float* Z, int64_t ldz, const int32_t* ids, const int32_t* rank, int64_t rows, int K,
                            float* zs, hipStream_t s) {
  const int64_t n = rows * K;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zs_from_z_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, Z, ldz, ids, rank, rows, K,
                     zs);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_mask_count(const uint8_t* mask, int64_t N, void* scal, hipStream_t s) {
  hipLaunchKernelGGL(mask_count_kernel, dim3(1), dim3(1024), 0, s, mask, N, (Scalars*)scal);
  return hipGetLastError();
}

hipError_t launch_row_stats(Dtype g_dt, const RowArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (g_dt == DT_BF16)
    hipLaunchKernelGGL(row_stats_kernel<__bf16>, dim3((unsigned)a.rows), dim3(kRowThreads), 0, s, a);
  else
    hipLaunchKernelGGL(row_stats_kernel<float>, dim3((unsigned)a.rows), dim3(kRowThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dense(Dtype g_dt, const RowArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.V + 63) / 64), (unsigned)((a.rows + 63) / 64));
  if (g_dt == DT_BF16)
    hipLaunchKernelGGL(dense_kernel<__bf16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(dense_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scatter(Dtype g_dt, const RowArgs& a, hipStream_t s) {
  const int64_t n = a.rows * a.K;
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (g_dt == DT_BF16)
    hipLaunchKernelGGL(scatter_kernel<__bf16>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(scatter_kernel<float>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_partials_from_z(Dtype g_dt, const float* Z, int64_t ldz, int64_t rows, int64_t V, float2* part,
                                  int n_slices, void* P, int64_t pblk, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid(n_slices, (unsigned)rows);
  if (g_dt == DT_BF16)
    hipLaunchKernelGGL(partials_from_z_kernel<__bf16>, grid, dim3(128), 0, s, Z, ldz, V, part, n_slices,
                       (__bf16*)P, pblk);
  else
    hipLaunchKernelGGL(partials_from_z_kernel<float>, grid, dim3(128), 0, s, Z, ldz, V, part, n_slices, (float*)P,
                       pblk);
  return hipGetLastError();
}

hipError_t launch_untile(Dtype g_dt, const void* P, int64_t pblk, int64_t rows, int64_t V, void* out,
                         hipStream_t s) {
  const int64_t n = rows * V;
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (g_dt == DT_BF16)
    hipLaunchKernelGGL(untile_kernel<__bf16>, dim3(blocks), dim3(256), 0, s, (const __bf16*)P, pblk, rows, V,
                       (__bf16*)out);
  else
    hipLaunchKernelGGL(untile_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)P, pblk, rows, V,
                       (float*)out);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* kl, int64_t N, const void* scal, float* out_loss, hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1024), 0, s, kl, N, (const Scalars*)scal, out_loss);
  return hipGetLastError();
}

}  // namespace ckl
