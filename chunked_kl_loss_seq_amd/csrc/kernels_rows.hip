// Per-token kernels of the fused chunked KL loss: valid-token count, the row
// pass over a chunk of logits (log-normaliser, teacher softmax over the cached
// top-K, gather, KL, in-place logit gradient and top-K scatter) and the final
// loss reduction.
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
#include <hip/hip_runtime.h>
#include <math.h>

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
};

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

// Make every global access this thread issued complete before the barrier
// that follows, so that other waves may overwrite those bytes after it.
__device__ inline void drain_memory() { __builtin_amdgcn_s_waitcnt(0); }

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
  }
}

// ------------------------------------------------------------------ row pass
// One workgroup per token row.  In the bf16 form the gradient row (bf16) is
// written over the first half of the bytes of its own fp32 logit row.  The row
// is walked in segments of 2048 logits: every thread reads its 8 logits of a
// segment and converts them, the workgroup synchronises, and only then are
// the 16-byte gradient pieces of that segment stored; they overwrite logits of
// earlier or the same segment only, all of which have been read.
template <bool G_BF16>
__global__ void __launch_bounds__(kRowThreads) row_kernel(RowArgs a) {
  constexpr int NT = kRowThreads;
  __shared__ float red[2 * (NT / 64)];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  float* zrow = a.Z + r * a.ldz;
  const Scalars* sc = (const Scalars*)a.scal;
  const float scale = sc ? sc->scale : a.scale_value;
  const bool valid = a.mask == nullptr || a.mask[r] != 0;
  const float w = valid ? scale : 0.f;

  // student log-normaliser from the per-slice partials
  float m = -INFINITY, s = 0.f;
  const float2* prow = a.part + r * a.n_slices;
  for (int p = tid; p < a.n_slices; p += NT) {
    const float2 q = prow[p];
    lse_merge(m, s, q.x, q.y);
  }
  block_lse_merge<NT>(m, s, red);
  const float lse = m + logf(s);

  // teacher softmax over the cached logits, gather, KL, scatter values
  const int K = a.K;
  float tv[kKPT], gv[kKPT];
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
    gv[q] = 0.f;
    if (k < K) {
      const float lpt = tv[q] - lse_t;
      const float pt = __expf(lpt);
      const float zg = zrow[iv[q]];
      klp += pt * (lpt - (zg - lse));
      gv[q] = valid ? w * (__expf(zg - lse) - pt) : 0.f;
      if (a.zg_dbg) {
        a.zg_dbg[r * K + k] = zg;
        a.sid_dbg[r * K + k] = iv[q];
      }
    }
  }
  const float kl = block_sum<NT>(klp, red);
  drain_memory();
  __syncthreads();

  // dense gradient pass, in place
  const int64_t V = a.V;
  const int64_t vpad = (V + 7) / 8 * 8;
  if constexpr (G_BF16) {
    typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
    __bf16* grow = (__bf16*)zrow;
    const int64_t nseg = (vpad + 8 * NT - 1) / (8 * NT);
    f32x4 x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
    int64_t j = (int64_t)tid * 8;
    if (valid && j < V) {
      x0 = *(const f32x4*)(zrow + j);
      x1 = *(const f32x4*)(zrow + j + 4);
    }
    for (int64_t sg = 0; sg < nseg; ++sg) {
      j = sg * 8 * NT + (int64_t)tid * 8;
      bf16x8 g;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float z = e < 4 ? x0[e] : x1[e - 4];
        const float v = (valid && j + e < V) ? w * __expf(z - lse) : 0.f;
        g[e] = (__bf16)v;
      }
      const int64_t jn = j + 8 * NT;
      if (valid && sg + 1 < nseg && jn < V) {
        x0 = *(const f32x4*)(zrow + jn);
        x1 = *(const f32x4*)(zrow + jn + 4);
      }
      // The converted values must exist (so this segment's logits have been
      // read) before the barrier; the next segment's loads may stay in flight,
      // their bytes are not stored to before the next barrier.
      u32x4 gbits = __builtin_bit_cast(u32x4, g);
      asm volatile("" ::"v"(gbits.x), "v"(gbits.y), "v"(gbits.z), "v"(gbits.w));
      __syncthreads();
      if (j < vpad) *(u32x4*)(grow + j) = gbits;
    }
  } else {
    for (int64_t j = (int64_t)tid * 4; j < vpad; j += 4 * NT) {
      f32x4 x = {0, 0, 0, 0};
      if (valid && j < V) x = *(const f32x4*)(zrow + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (valid && j + e < V) ? w * __expf(x[e] - lse) : 0.f;
      *(f32x4*)(zrow + j) = x;
    }
  }
  drain_memory();
  __syncthreads();

  // the cached ids get the exact combined value w (p_S - p_T)
  if (valid) {
#pragma unroll
    for (int q = 0; q < kKPT; ++q) {
      const int k = tid + q * NT;
      if (k < K) {
        if constexpr (G_BF16)
          ((__bf16*)zrow)[iv[q]] = (__bf16)gv[q];
        else
          zrow[iv[q]] = gv[q];
      }
    }
  }
  if (tid == 0) {
    a.kl_out[r] = valid ? kl : 0.f;
    a.lse_out[r] = lse;
  }
}

// ------------------------------------------------------------------ debug partials
__global__ void __launch_bounds__(128) partials_from_z_kernel(const float* __restrict__ Z, int64_t ldz, int64_t V,
                                                              float2* __restrict__ part, int n_slices) {
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
  float s = wave_sum(ok ? __expf(z - m) : 0.f);
  if ((threadIdx.x & 63) == 0) red[2 + (threadIdx.x >> 6)] = s;
  __syncthreads();
  if (threadIdx.x == 0) part[r * n_slices + slice] = make_float2(m, red[2] + red[3]);
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

hipError_t launch_mask_count(const uint8_t* mask, int64_t N, void* scal, hipStream_t s) {
  hipLaunchKernelGGL(mask_count_kernel, dim3(1), dim3(1024), 0, s, mask, N, (Scalars*)scal);
  return hipGetLastError();
}

hipError_t launch_rows(Dtype g_dt, const RowArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (g_dt == DT_BF16)
    hipLaunchKernelGGL(row_kernel<true>, dim3((unsigned)a.rows), dim3(kRowThreads), 0, s, a);
  else
    hipLaunchKernelGGL(row_kernel<false>, dim3((unsigned)a.rows), dim3(kRowThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_partials_from_z(const float* Z, int64_t ldz, int64_t rows, int64_t V, float2* part,
                                  int n_slices, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(partials_from_z_kernel, dim3(n_slices, (unsigned)rows), dim3(128), 0, s, Z, ldz, V, part,
                     n_slices);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* kl, int64_t N, const void* scal, float* out_loss, hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1024), 0, s, kl, N, (const Scalars*)scal, out_loss);
  return hipGetLastError();
}

}  // namespace ckl
