// Offline top-K cache writer: per row of teacher logits, the K largest values
// and their ids, by value descending and equal values by id ascending.
//
// The teacher runs once and only its K most likely predictions per position
// are stored ("A New Trick Slashes the Cost of Shrinking Giant AI Models",
// section "What did the researchers change?"; "Making Knowledge Distillation
// Cheap Enough to Run at Scale" (elseif.net), offline-cache paragraph).  The
// pages do not order equal logits; the order taken here is the stable one
// (lower id first), which makes the result unique.
//
// One workgroup per row, bound by reading the row (2 or 4 bytes per logit).
// Values are compared through an order-preserving unsigned key of their bits
// (-0 is keyed as +0; NaN is outside the supported inputs):
//  1. every thread takes the largest key of its strided share of the row;
//  2. t0 = the lower edge of the histogram bin (top 13 key bits) in which,
//     counting the maxima from the top, the K-th one falls; those K maxima
//     are K distinct elements, so at least K keys are >= t0;
//  3. the elements with key >= t0 are collected into LDS as (key, id) pairs;
//     each thread kept the largest value of each of its 16-byte chunks (bf16
//     rows) or of every group of 8 of them (fp32 rows), so only the chunks or
//     groups that reach t0 are read again (a few percent of the row);
//  4. ordered by (key descending, id ascending): each pair's place is the
//     number of larger pairs (a bitonic sort when more pairs than threads).
// When more than kCap elements reach t0 (many equal values near the top) or
// K exceeds the thread count, an exact path takes over: a binary search over
// the key range finds the K-th largest key T, the elements above T are
// collected, and the elements equal to T are taken in id order with one
// block-wide scan per run of ids until K are held.
#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace ckl {

namespace {

constexpr int kTopkThreads = 512;
constexpr int kCap = 4096;  // (key, id) pairs held in LDS (at least the largest K)
constexpr int kHistBits = 13;
constexpr int kHistBins = 1 << kHistBits;
static_assert(kHistBins * 4 <= kCap * 8, "the histogram lives in the candidate store");
static_assert(kHistBins % kTopkThreads == 0, "whole bins per thread");
static_assert(kCap >= kMaxK, "the exact path holds K pairs");

template <typename T>
struct Key;
template <>
struct Key<__bf16> {
  static constexpr int kBits = 16;
  __device__ static inline uint32_t of(__bf16 v) {
    uint32_t b = __builtin_bit_cast(uint16_t, v);
    if (b == 0x8000u) b = 0;
    return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
  }
};
template <>
struct Key<float> {
  static constexpr int kBits = 32;
  __device__ static inline uint32_t of(float v) {
    uint32_t b = __builtin_bit_cast(uint32_t, v);
    if (b == 0x80000000u) b = 0;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Element i of a 16-byte chunk, taken out by bit casts (no type punning
// through pointers).
__device__ inline __bf16 chunk_elem(const u32x4_t& v, int i, __bf16*) {
  const uint32_t w = v[i >> 1];
  return __builtin_bit_cast(__bf16, (uint16_t)((i & 1) ? (w >> 16) : (w & 0xFFFFu)));
}
__device__ inline float chunk_elem(const u32x4_t& v, int i, float*) {
  const uint32_t w = v[i];  // a scalar first: bit-casting the subscript itself read lane 0
  return __builtin_bit_cast(float, w);
}

// Largest value of a 16-byte chunk as fp32 (bf16 halves widened by a mask or
// a shift: exact).  The streaming passes work on values, which costs about
// one max instruction per element; keys are formed only for the threshold and
// for the few elements that reach it.
__device__ inline float chunk_max(const u32x4_t& v, __bf16*) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[i];
    const float hi = __builtin_bit_cast(float, w & 0xFFFF0000u);
    const float lo = __builtin_bit_cast(float, w << 16);
    m = fmaxf(m, fmaxf(hi, lo));
  }
  return m;
}
__device__ inline float chunk_max(const u32x4_t& v, float*) {
  const uint32_t a = v[0], b = v[1], c = v[2], d = v[3];
  return fmaxf(fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)),
               fmaxf(__builtin_bit_cast(float, c), __builtin_bit_cast(float, d)));
}

// Key of a value held exactly in fp32 (a widened bf16 or an fp32 element).
template <typename T>
__device__ inline uint32_t key_of_value(float v) {
  if constexpr (sizeof(T) == 2)
    return Key<__bf16>::of(__builtin_bit_cast(__bf16, (uint16_t)(__builtin_bit_cast(uint32_t, v) >> 16)));
  else
    return Key<float>::of(v);
}

// Per-thread maxima kept from the first pass so that the second pass reads
// again only what can reach the threshold.  bf16 rows keep the maximum of
// every chunk (exact in bf16, two per register; a re-read then touches one
// 16-byte chunk instead of eight scattered ones); fp32 rows keep the maximum
// of every group of 8 chunks.  Rows with more chunks per thread than kept
// here are scanned again whole.
template <typename T>
struct GroupMax;
template <>
struct GroupMax<__bf16> {
  static constexpr int kGroup = 1;    // chunks per group
  static constexpr int kGroups = 64;  // groups per thread: rows up to 262,144 bf16
  uint32_t w[kGroups / 2];
  // m holds a bf16 value exactly (or -inf)
  __device__ inline void set(int g, float m) {
    const uint32_t b = __builtin_bit_cast(uint32_t, m) >> 16;
    w[g >> 1] = (g & 1) ? ((w[g >> 1] & 0xFFFFu) | (b << 16)) : b;
  }
  __device__ inline float get(int g) const {
    const uint32_t b = (g & 1) ? (w[g >> 1] & 0xFFFF0000u) : (w[g >> 1] << 16);
    return __builtin_bit_cast(float, b);
  }
};
template <>
struct GroupMax<float> {
  static constexpr int kGroup = 8;
  static constexpr int kGroups = 16;  // rows up to 262,144 fp32
  float w[kGroups];
  __device__ inline void set(int g, float m) { w[g] = m; }
  __device__ inline float get(int g) const { return w[g]; }
};

// The value whose key is t, for t above the key of -inf (below it the bit
// patterns are NaNs): the keys invert back to bit patterns.
template <typename T>
__device__ inline float value_of_key(uint32_t t) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t b = (t & 0x8000u) ? (t & 0x7FFFu) : (~t & 0xFFFFu);
    return __builtin_bit_cast(float, b << 16);
  } else {
    const uint32_t b = (t & 0x80000000u) ? (t & 0x7FFFFFFFu) : ~t;
    return __builtin_bit_cast(float, b);
  }
}

// (key, id) packed so that a larger number means an earlier place in the
// answer: key descending, then id ascending.
__device__ inline uint64_t pack(uint32_t key, uint32_t id) { return ((uint64_t)key << 32) | (0xFFFFFFFFu - id); }
__device__ inline uint32_t unpack_id(uint64_t c) { return 0xFFFFFFFFu - (uint32_t)c; }

// Sort a[0, n) descending (n a power of two), all threads of the block.
__device__ inline void bitonic_desc(uint64_t* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kTopkThreads) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t x = a[i], y = a[l];
          const bool first_half_desc = (i & k) == 0;
          if (first_half_desc ? (x < y) : (x > y)) {
            a[i] = y;
            a[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ inline uint32_t block_sum(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < kTopkThreads / 64; ++i) t += red[i];
  return t;
}

// Sum of v over the threads after this one (thread order).
__device__ inline uint32_t block_suffix_excl(uint32_t v, uint32_t* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;  // becomes the sum over lanes >= lane of this wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_down(x, o);
    if (lane + o < 64) x += y;
  }
  __syncthreads();
  if (lane == 0) red[w] = x;
  __syncthreads();
  uint32_t later = 0;
#pragma unroll
  for (int i = 0; i < kTopkThreads / 64; ++i) later += i > w ? red[i] : 0;
  return later + x - v;
}

// Exclusive rank of this thread's flag among the block's set flags (thread
// order) and the total number set.
__device__ inline uint32_t block_rank(bool f, uint32_t* red, uint32_t* total) {
  const uint64_t bal = __ballot(f);
  const uint32_t in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = (uint32_t)__popcll(bal);
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kTopkThreads / 64; ++i) {
    before += i < w ? red[i] : 0;
    all += red[i];
  }
  *total = all;
  return before + in_wave;
}

// Visit every element of a row as (key, id): 16-byte loads when the row is
// 16-byte aligned and a whole number of 16-byte chunks (then many loads per
// thread are in flight at once), element loads otherwise.
template <typename T, typename F>
__device__ inline void for_each_key(const T* row, int64_t V, bool vec, F&& fn) {
  if (vec) {
    constexpr int EPC = 16 / (int)sizeof(T);
    const u32x4_t* p = (const u32x4_t*)row;
    const int64_t chunks = V / EPC;
#pragma unroll 4
    for (int64_t c = threadIdx.x; c < chunks; c += kTopkThreads) {
      const u32x4_t v = p[c];
#pragma unroll
      for (int i = 0; i < EPC; ++i) fn(Key<T>::of(chunk_elem(v, i, (T*)nullptr)), c * EPC + i);
    }
  } else {
#pragma unroll 8
    for (int64_t e = threadIdx.x; e < V; e += kTopkThreads) fn(Key<T>::of(row[e]), e);
  }
}

// The input value of a held pair, rebuilt from its key; only a zero is read
// back from the row, since -0 and +0 share one key and the value must keep
// the input's sign.
template <typename T>
__device__ inline float value_out(uint64_t c, const T* row, uint32_t id) {
  const uint32_t key = (uint32_t)(c >> 32);
  if (key == Key<T>::of((T)0.f)) return (float)row[id];
  return value_of_key<T>(key);
}

template <typename T>
__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const T* __restrict__ x, int64_t V, int K,
                                                           int32_t* __restrict__ ids_out,
                                                           float* __restrict__ vals_out) {
  __shared__ uint64_t cand[kCap];
  __shared__ uint32_t red[kTopkThreads / 64];
  __shared__ uint32_t count, t0_s;
  const int tid = threadIdx.x;
  const T* row = x + (int64_t)blockIdx.x * V;
  const bool vec = ((uintptr_t)row % 16 == 0) && ((V * (int64_t)sizeof(T)) % 16 == 0);
  constexpr int kEPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  const u32x4_t* p = (const u32x4_t*)row;
  const uint32_t chunks = vec ? (uint32_t)(V / kEPC) : 0u;
  typedef GroupMax<T> GM;
  constexpr int kGroup = GM::kGroup, kGroups = GM::kGroups;
  // rows of at most kGroups x kGroup chunks per thread keep each group's maximum
  const bool grouped = vec && chunks <= (uint32_t)(kGroups * kGroup * kTopkThreads);
  GM gmax;

  bool exact = K > kTopkThreads;
  uint32_t n_held = 0;
  if (!exact) {
    // 1. largest key of this thread's share
    uint32_t mk = 0;  // 0 is below every element's key: a thread with no element
    if (grouped) {
      float mv = -INFINITY;
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        float gm = -INFINITY;
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
          // loads clamped into the row and always issued, so that a group's
          // loads are in flight together; chunks past the row are masked
          const uint32_t c = (uint32_t)tid + (uint32_t)((g * kGroup + j) * kTopkThreads);
          const float m = chunk_max(p[c < chunks ? c : chunks - 1], (T*)nullptr);
          gm = fmaxf(gm, c < chunks ? m : -INFINITY);
        }
        gmax.set(g, gm);
        mv = fmaxf(mv, gm);
      }
      mk = (uint32_t)tid < chunks ? key_of_value<T>(mv) : 0u;
    } else if (vec) {
      float mv = -INFINITY;
      bool any = false;
#pragma unroll 4
      for (uint32_t c = tid; c < chunks; c += kTopkThreads) {
        mv = fmaxf(mv, chunk_max(p[c], (T*)nullptr));
        any = true;
      }
      mk = any ? key_of_value<T>(mv) : 0u;
    } else {
      for_each_key(row, V, vec, [&](uint32_t k, int64_t) { mk = max(mk, k); });
    }
    // 2. t0 = the lower edge of the histogram bin (top 13 key bits) of the
    //    maxima where, counting from the top, K maxima are reached: at least
    //    K maxima, so K distinct elements, have key >= t0
    uint32_t* hist = (uint32_t*)cand;  // free until the candidates are collected
    constexpr int kShift = Key<T>::kBits - kHistBits;
    for (int i = tid; i < kHistBins; i += kTopkThreads) hist[i] = 0;
    if (tid == 0) count = 0;
    __syncthreads();
    atomicAdd(&hist[mk >> kShift], 1u);
    __syncthreads();
    constexpr int kPer = kHistBins / kTopkThreads;  // bins per thread, thread t owns [kPer t, kPer t + kPer)
    uint32_t mine = 0;
#pragma unroll
    for (int b = 0; b < kPer; ++b) mine += hist[kPer * tid + b];
    const uint32_t above = block_suffix_excl(mine, red);  // maxima in the bins of higher threads
    if (above < (uint32_t)K && above + mine >= (uint32_t)K) {
      uint32_t c = above;
      for (int b = kPer - 1; b >= 0; --b) {
        c += hist[kPer * tid + b];
        if (c >= (uint32_t)K) {
          t0_s = (uint32_t)(kPer * tid + b) << kShift;
          break;
        }
      }
    }
    __syncthreads();
    const uint32_t t0 = t0_s;
    // 3. every element with key >= t0
    auto hold = [&](uint32_t k, int64_t e) {
      if (k >= t0) {
        const uint32_t slot = atomicAdd(&count, 1u);
        if (slot < (uint32_t)kCap) cand[slot] = pack(k, (uint32_t)e);
      }
    };
    // a chunk (or group) can hold such an element only if its largest value
    // reaches the value of t0.  A t0 at or below the key of -inf (its bit
    // pattern would be a NaN) admits every element; -0 compares equal to +0.
    const float v0 = t0 <= Key<T>::of((T)-INFINITY) ? -INFINITY : value_of_key<T>(t0);
    auto scan_chunk = [&](uint32_t c) {
      const u32x4_t v = p[c];
      if (chunk_max(v, (T*)nullptr) >= v0) {
#pragma unroll
        for (int i = 0; i < kEPC; ++i)
          hold(Key<T>::of(chunk_elem(v, i, (T*)nullptr)), (int64_t)c * kEPC + i);
      }
    };
    if (grouped) {
      // only the groups whose maximum (kept from step 1) reaches t0 are read
      // again: a bit mask of them first (register indices stay static), then
      // one pass over its set bits
      static_assert(kGroups <= 64, "one bit per group");
      uint64_t todo = 0;
#pragma unroll
      for (int g = 0; g < kGroups; ++g) todo |= (uint64_t)(gmax.get(g) >= v0) << g;
      while (todo) {
        const int g = __builtin_ctzll(todo);
        todo &= todo - 1;
        for (int j = 0; j < kGroup; ++j) {
          const uint32_t c = (uint32_t)tid + (uint32_t)((g * kGroup + j) * kTopkThreads);
          if (c < chunks) scan_chunk(c);
        }
      }
    } else if (vec) {
#pragma unroll 4
      for (uint32_t c = tid; c < chunks; c += kTopkThreads) scan_chunk(c);
    } else {
      for_each_key(row, V, vec, hold);
    }
    __syncthreads();
    n_held = count;
    // every thread has read the count before the exact path may reset it
    __syncthreads();
    exact = n_held > (uint32_t)kCap;
  }

  int n = K;
  if (!exact) {
    n = (int)n_held;
  } else {
    // exact path: T = the K-th largest key, by binary search over the key range
    uint64_t lo = 0, hi = (Key<T>::kBits == 32) ? 0xFFFFFFFFull : 0xFFFFull;
    while (lo < hi) {
      const uint64_t mid = lo + (hi - lo + 1) / 2;
      uint32_t c = 0;
      for (int64_t e = tid; e < V; e += kTopkThreads) c += Key<T>::of(row[e]) >= (uint32_t)mid;
      if (block_sum(c, red) >= (uint32_t)K)
        lo = mid;
      else
        hi = mid - 1;
    }
    const uint32_t T0 = (uint32_t)lo;
    if (tid == 0) count = 0;
    __syncthreads();
    // the elements above T (fewer than K of them)
    for (int64_t e = tid; e < V; e += kTopkThreads) {
      const uint32_t k = Key<T>::of(row[e]);
      if (k > T0) cand[atomicAdd(&count, 1u)] = pack(k, (uint32_t)e);
    }
    __syncthreads();
    const uint32_t above = count;
    // the elements equal to T, lowest ids first, until K are held
    uint32_t taken = 0, need = (uint32_t)K - above;
    for (int64_t base = 0; need > 0 && base < V; base += kTopkThreads) {
      const int64_t e = base + tid;
      const bool f = e < V && Key<T>::of(row[e]) == T0;
      uint32_t total = 0;
      const uint32_t rank = block_rank(f, red, &total);
      if (f && rank < need) cand[above + taken + rank] = pack(T0, (uint32_t)e);
      const uint32_t got = total < need ? total : need;
      taken += got;
      need -= got;
    }
    __syncthreads();
  }

  // 4. order the held pairs and write the first K.  The packed pairs are
  //    distinct, so a pair's place is the number of larger pairs: up to one
  //    pair per thread that count is cheaper than a sort.
  int32_t* io = ids_out + (int64_t)blockIdx.x * K;
  float* vo = vals_out + (int64_t)blockIdx.x * K;
  if (n <= kTopkThreads) {
    if (tid < n) {
      const uint64_t c = cand[tid];
      int place = 0;
      for (int i = 0; i < n; ++i) place += cand[i] > c;
      if (place < K) {
        const uint32_t id = unpack_id(c);
        io[place] = (int32_t)id;
        vo[place] = value_out<T>(c, row, id);
      }
    }
    return;
  }
  int p2 = 1;
  while (p2 < n) p2 <<= 1;
  for (int i = n + tid; i < p2; i += kTopkThreads) cand[i] = 0;  // below every real pair
  __syncthreads();
  bitonic_desc(cand, p2);
  for (int k = tid; k < K; k += kTopkThreads) {
    const uint32_t id = unpack_id(cand[k]);
    io[k] = (int32_t)id;
    vo[k] = value_out<T>(cand[k], row, id);
  }
}

}  // namespace

hipError_t launch_topk(Dtype dt, const void* x, int64_t N, int64_t V, int64_t K, int32_t* ids, float* vals,
                       hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (dt == DT_BF16)
    hipLaunchKernelGGL(topk_kernel<__bf16>, dim3((unsigned)N), dim3(kTopkThreads), 0, s, (const __bf16*)x, V,
                       (int)K, ids, vals);
  else
    hipLaunchKernelGGL(topk_kernel<float>, dim3((unsigned)N), dim3(kTopkThreads), 0, s, (const float*)x, V, (int)K,
                       ids, vals);
  return hipGetLastError();
}

}  // namespace ckl
