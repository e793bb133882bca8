// Launchers of the two gradient contractions (dH, dW), the tiled copy and the
// split-K reduce.  The logits contraction has its own unit (kernels_logits.hip).
#include "gemm_core.hpp"
#include "launch.hpp"

namespace ckl {

constexpr int kGroupM = 4;

// bf16: 256-wide tiles along d (8 waves of 128 x 64), measured faster than
// 192-wide ones even where 192 divides d and 256 does not.  fp32 fragments are
// twice as wide: 192 where it divides d (and 256 does not), else 128, whose
// 64 x 64 wave tiles leave the loop spill-free (256 x 256 spilled).
int d_tile(Dtype dt, int64_t d) {
  if (dt == DT_BF16) return 256;
  return (d % 192 == 0 && d % 256 != 0) ? 192 : 128;
}

int dh_splits(Dtype dt, int64_t rows, int64_t d, int64_t V) {
  // Pick the k-split count that best fills whole waves of 256 workgroups:
  // 1..8, or up to 32 when 8 splits do not fill one wave (small chunks, whose
  // slabs are small).  Each split keeps at least 8 k-steps, and only counts
  // that cut the k-steps into exactly that many runs are taken.
  const int64_t tiles = ((rows + 255) / 256) * ((d + d_tile(dt, d) - 1) / d_tile(dt, d));
  const int64_t ksteps = (V + (dt == DT_BF16 ? 63 : 31)) / (dt == DT_BF16 ? 64 : 32);
  const int max_s = tiles * 8 < 256 ? 32 : 8;
  int best = 1;
  double best_eff = -1.0;
  for (int s = 1; s <= max_s; ++s) {
    if (s > 1 && ksteps / s < 8) break;
    const int64_t per = (ksteps + s - 1) / s;
    if ((ksteps + per - 1) / per != s) continue;
    const double waves = (double)tiles * s / 256.0;
    const double eff = waves / (double)((int64_t)(waves + 0.999999));
    if (eff > best_eff + 0.02) {
      best_eff = eff;
      best = s;
    }
  }
  return best;
}

int dh_fit_splits(Dtype dt, int64_t V, int s) {
  const int64_t ksteps = (V + (dt == DT_BF16 ? 63 : 31)) / (dt == DT_BF16 ? 64 : 32);
  if (s < 1) return 1;
  const int64_t per = (ksteps + s - 1) / s;
  return (int)((ksteps + per - 1) / per);  // at most s, and cuts the k-steps into exactly that many runs
}

hipError_t launch_dh(Dtype dt, const void* G, int64_t gblk, const void* Wt, int64_t V, int64_t d, int64_t rows,
                     float* slab, int splits, const int* live, hipStream_t s) {
  const int bn = d_tile(dt, d);
  const int bk = dt == DT_BF16 ? 64 : 32;
  GemmParams p{};
  p.live = live;
  p.a = Operand{G, 0, rows, V, gblk};  // tiled: storage row = token, column = vocabulary id
  p.b = Operand{Wt, 0, d, V, tile_row_stride(d)};  // tiled: storage row = vocabulary id (k), column = d (n)
  p.tiles_m = cdiv64(rows, 256);
  p.tiles_n = cdiv64(d, bn);
  p.k_tiles = cdiv64(V, bk);
  p.k_tiles_per_split = cdiv64(p.k_tiles, splits);
  p.splits = cdiv64(p.k_tiles, p.k_tiles_per_split);
  p.group_m = kGroupM;
  p.out = slab;
  p.ldo = d;
  p.split_stride = rows * d;
  p.valid_m = rows;
  p.valid_n = d;
  if (p.splits != splits) return hipErrorInvalidValue;
  if (dt == DT_BF16) return launch_gemm<__bf16, 256, 256, 2, 4, true, false, EPI_SLAB, 128, 2>(p, s);
  if (bn == 192) return launch_gemm<float, 256, 192, 4, 2, true, false, EPI_SLAB, 128, 2>(p, s);
  return launch_gemm<float, 256, 128, 4, 2, true, false, EPI_SLAB, 128, 2>(p, s);
}

hipError_t launch_dw(Dtype dt, const void* G, int64_t gblk, const void* Hc, int64_t V, int64_t d, int64_t rows,
                     float* dW, int beta, const int* live, hipStream_t s) {
  const int bn = d_tile(dt, d);
  const int bk = dt == DT_BF16 ? 64 : 32;
  GemmParams p{};
  p.live = live;
  p.a = Operand{G, 0, V, rows, gblk};  // tiled: storage row = token (k), column = vocabulary id (m)
  p.b = Operand{Hc, d, d, rows, 0};
  p.tiles_m = cdiv64(V, 256);
  p.tiles_n = cdiv64(d, bn);
  p.k_tiles = cdiv64(rows, bk);
  p.splits = 1;
  p.k_tiles_per_split = p.k_tiles;
  p.group_m = 1;  // all d-tiles of a vocabulary row-block together: they share the G^T slab
  p.out = dW;
  p.ldo = d;
  p.valid_m = V;
  p.valid_n = d;
  p.beta = beta;
  if (dt == DT_BF16) return launch_gemm<__bf16, 256, 256, 2, 4, false, false, EPI_ACCUM, 128, 2>(p, s);
  if (bn == 192) return launch_gemm<float, 256, 192, 4, 2, false, false, EPI_ACCUM, 128, 2>(p, s);
  return launch_gemm<float, 256, 128, 4, 2, false, false, EPI_ACCUM, 128, 2>(p, s);
}

// ---------------------------------------------------------------- tiled copy
template <typename T>
__global__ void __launch_bounds__(256) tile_copy_kernel(const T* __restrict__ src, int64_t rows, int64_t cols,
                                                       T* __restrict__ dst, int64_t dblk) {
  constexpr int EPC = 16 / sizeof(T);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = cols / EPC;
  if (i >= rows * per_row) return;
  const int64_t r = i / per_row, c = (i - r * per_row) * EPC;
  const u32x4 v = *(const u32x4*)(src + r * cols + c);
  *(u32x4*)(dst + (r >> 6) * dblk + (c >> 6) * 4096 + (r & 63) * 64 + (c & 63)) = v;
}

hipError_t launch_tile_copy(Dtype dt, const void* src, int64_t rows, int64_t cols, void* dst, hipStream_t s) {
  const int64_t n = rows * cols / (dt == DT_BF16 ? 8 : 4);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(tile_copy_kernel<__bf16>, dim3(blocks), dim3(256), 0, s, (const __bf16*)src, rows, cols,
                       (__bf16*)dst, tile_row_stride(cols));
  else
    hipLaunchKernelGGL(tile_copy_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)src, rows, cols,
                       (float*)dst, tile_row_stride(cols));
  return hipGetLastError();
}

// ---------------------------------------------------------------- split-K reduce
// Thread: 4 consecutive dH elements of one row (d % 8 == 0).  With pos, the
// output row j reads slab row pos[j] (a compacted chunk) or writes zeros.
template <typename TO>
__global__ void __launch_bounds__(256) dh_reduce_kernel(const float* __restrict__ slab, int splits, int64_t count,
                                                       int64_t d, const int* __restrict__ pos,
                                                       TO* __restrict__ out) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= count) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int64_t src = i4;
  bool live = true;
  if (pos != nullptr) {
    const int64_t j = i4 / d;
    const int p = pos[j];
    live = p >= 0;
    src = (int64_t)p * d + (i4 - j * d);
  }
  if (live) {
    acc = *(const f32x4*)(slab + src);
    for (int s = 1; s < splits; ++s) acc += *(const f32x4*)(slab + (int64_t)s * count + src);
  }
  if constexpr (sizeof(TO) == 4) {
    *(f32x4*)((float*)out + i4) = acc;
  } else {
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
    bf16x4 v = {(__bf16)acc.x, (__bf16)acc.y, (__bf16)acc.z, (__bf16)acc.w};
    *(bf16x4*)((__bf16*)out + i4) = v;
  }
}

hipError_t launch_dh_reduce(Dtype dt, const float* slab, int splits, int64_t rows, int64_t d, const int* pos,
                            void* dH, hipStream_t s) {
  const int64_t count = rows * d;  // d % 8 == 0, so count % 4 == 0
  const int64_t blocks = (count / 4 + 255) / 256;
  if (dt == DT_BF16)
    hipLaunchKernelGGL(dh_reduce_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, s, slab, splits, count, d,
                       pos, (__bf16*)dH);
  else
    hipLaunchKernelGGL(dh_reduce_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, slab, splits, count, d,
                       pos, (float*)dH);
  return hipGetLastError();
}

}  // namespace ckl
