// MFMA GEMM engine for gfx950 (CDNA4), shared by the three contractions of the
// fused chunked KL loss:
//   logits    Z^T tile = W . H_c^T   (both operands contiguous along d)
//   dH        dH_c     = G . W       (G contiguous along V, W contiguous along d)
//   dW        dW      += G^T . H_c   (both operands contiguous along the token axis)
//
// One workgroup computes a BM x BN tile of D = A . B with WM x WN waves.  Each
// k-step stages a BK-deep slab of A and B through LDS (double buffered):
//   * an operand contiguous along k ("k-major") is kept as [row][128 bytes]
//     with a 16-byte-chunk XOR swizzle and read as one ds_read_b128 per MFMA
//     fragment;
//   * an operand contiguous along m or n ("mn-major") is kept as it lies in
//     memory, [k][row] with a 32-byte row pad, and read with ds_read_tr16_b64,
//     which hands each lane four k-consecutive 16-bit values of one column
//     (two reads per bf16 fragment).  fp32 mn-major operands use ds_read_b32.
// bf16 operands use v_mfma_f32_32x32x16_bf16; fp32 operands use
// v_mfma_f32_32x32x2_f32 over the same LDS layout: a fragment holds the
// 8 k-values k0 + 8h .. k0 + 8h + 7 of lane half h in both cases, and the
// fp32 path issues 8 MFMAs, one per element, which pair the same k on the A
// and B side.
//
// Accumulator layout of a 32x32 MFMA block (checked on gfx950): lane l, slot r
// holds D[(r/4)*8 + (l/32)*4 + r%4][l%32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckl {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One GEMM operand in global memory.  Element (mn, k) lives at
// ptr[mn * ld + k] when k-major and at ptr[k * ld + mn] when mn-major.
// Rows mn >= mn_ext and columns k >= k_ext read as zero.
struct Operand {
  const void* ptr;
  int64_t ld;
  int64_t mn_ext;
  int64_t k_ext;
};

enum EpilogueKind : int {
  EPI_LOGITS = 0,  // Z[n][m] = D[m][n] (fp32) + per (n, 128-row slice of m) (max, sum exp)
  EPI_SLAB = 1,    // out[m][n] = D[m][n] (fp32), one slab per k-split
  EPI_ACCUM = 2,   // out[m][n] = D[m][n] (beta = 0) or out[m][n] += D[m][n] (beta = 1)
};

struct GemmParams {
  Operand a, b;
  int tiles_m, tiles_n;  // output tiles
  int k_tiles;           // ceil(K / BK)
  int splits;            // k-splits; each covers k_tiles_per_split k-steps
  int k_tiles_per_split;
  int group_m;           // m-tiles per group in the tile order
  float* out;            // Z, slab base or dW
  int64_t ldo;
  int64_t split_stride;  // elements between k-split slabs (EPI_SLAB)
  int64_t valid_m, valid_n;  // stores are limited to m < valid_m, n < valid_n
  float2* part;          // EPI_LOGITS: partial (max, sum exp) per [n][slice]
  int n_slices;          // EPI_LOGITS: slices per row of part
  int beta;              // EPI_ACCUM
};

template <typename T>
struct ElemTraits;
template <>
struct ElemTraits<__bf16> {
  static constexpr int kBK = 64;  // k elements per 128-byte row
};
template <>
struct ElemTraits<float> {
  static constexpr int kBK = 32;
};

// ---------------------------------------------------------------- LDS layouts
template <typename T, int R, bool KMAJ>
struct TileLayout;

// k-major: [R rows][128 bytes], chunk c of row r stored at chunk c ^ (r & 7).
template <typename T, int R>
struct TileLayout<T, R, true> {
  static constexpr int kBytes = R * 128;
  __device__ static inline int off(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }
};

// mn-major: [BK k-rows][R * sizeof(T) + 32 bytes].  The 32-byte pad puts the
// four k-rows one ds_read_tr16_b64 group touches in distinct bank quarters.
template <typename T, int R>
struct TileLayout<T, R, false> {
  static constexpr int kPitch = R * (int)sizeof(T) + 32;
  static constexpr int kBytes = ElemTraits<T>::kBK * kPitch;
  __device__ static inline int off(int krow, int chunk) { return krow * kPitch + chunk * 16; }
};

// ---------------------------------------------------------------- global -> registers
// Each thread carries NCH 16-byte chunks of the tile in flight.
template <typename T, int R, int NT, bool KMAJ>
struct TileLoader {
  static constexpr int kEPC = 16 / (int)sizeof(T);          // elements per 16-byte chunk
  static constexpr int kChunks = R * 8;                      // 128 bytes of k per row, or BK rows of R
  static constexpr int kNCH = kChunks / NT;
  static_assert(kChunks % NT == 0, "tile chunks must divide evenly over the workgroup");
  static constexpr int kCPR = KMAJ ? 8 : R * (int)sizeof(T) / 16;  // chunks per stored row

  __device__ static inline void load(u32x4 (&r)[kNCH], const Operand& o, int64_t mn0, int64_t k0, int tid) {
    const T* base = (const T*)o.ptr;
#pragma unroll
    for (int i = 0; i < kNCH; ++i) {
      const int idx = tid + i * NT;
      const int srow = idx / kCPR, c = idx % kCPR;
      int64_t mn, k;
      if (KMAJ) {
        mn = mn0 + srow;
        k = k0 + (int64_t)c * kEPC;
      } else {
        k = k0 + srow;
        mn = mn0 + (int64_t)c * kEPC;
      }
      const bool ok = (mn < o.mn_ext) && (k < o.k_ext);
      const int64_t e = KMAJ ? (mn * o.ld + k) : (k * o.ld + mn);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *(const u32x4*)(base + e);
      r[i] = v;
    }
  }

  __device__ static inline void store(char* lds, const u32x4 (&r)[kNCH], int tid) {
#pragma unroll
    for (int i = 0; i < kNCH; ++i) {
      const int idx = tid + i * NT;
      const int srow = idx / kCPR, c = idx % kCPR;
      *(u32x4*)(lds + TileLayout<T, R, KMAJ>::off(srow, c)) = r[i];
    }
  }
};

// ---------------------------------------------------------------- LDS -> MFMA fragments
template <typename T>
struct Frag;
template <>
struct Frag<__bf16> {
  typedef bf16x8 type;
};
template <>
struct Frag<float> {
  typedef f32x8 type;
};

// Fragment of 32 rows (rows row0 .. row0+31 of the tile) x 16 k (sub-step kk).
template <typename T, int R, bool KMAJ>
__device__ inline typename Frag<T>::type load_frag(const char* lds, int row0, int kk, int lane);

template <typename T, int R, bool KMAJ>
__device__ inline typename Frag<T>::type load_frag(const char* lds, int row0, int kk, int lane) {
  typedef TileLayout<T, R, KMAJ> L;
  const int h = lane >> 5;
  if constexpr (KMAJ) {
    const int row = row0 + (lane & 31);
    if constexpr (sizeof(T) == 2) {
      u32x4 v = *(const u32x4*)(lds + L::off(row, 2 * kk + h));
      return __builtin_bit_cast(bf16x8, v);
    } else {
      u32x4 v0 = *(const u32x4*)(lds + L::off(row, 4 * kk + 2 * h));
      u32x4 v1 = *(const u32x4*)(lds + L::off(row, 4 * kk + 2 * h + 1));
      f32x8 f;
      f.lo = __builtin_bit_cast(f32x4, v0);
      f.hi = __builtin_bit_cast(f32x4, v1);
      return f;
    }
  } else {
    if constexpr (sizeof(T) == 2) {
      // 16-lane group g: column block (g & 1) * 16, k block (g >> 1) * 8.
      // Within the group, source lane 4j + p reads k-row j (+4 for the second
      // read) at columns 4p .. 4p+3; the transpose hands lane i column i.
      const int g = lane >> 4, i = lane & 15;
      const int krow = 16 * kk + (g >> 1) * 8 + (i >> 2);
      const int col = row0 + (g & 1) * 16 + 4 * (i & 3);
      const char* p0 = lds + krow * L::kPitch + col * 2;
      const char* p1 = p0 + 4 * L::kPitch;
      i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
      i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
      u32x4 v;
      u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      v.x = l2.x;
      v.y = l2.y;
      v.z = h2.x;
      v.w = h2.y;
      return __builtin_bit_cast(bf16x8, v);
    } else {
      const int col = row0 + (lane & 31);
      f32x8 f;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = *(const float*)(lds + (16 * kk + 8 * h + j) * L::kPitch + col * 4);
      return f;
    }
  }
}

__device__ inline f32x16 mfma_block(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16 mfma_block(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// ---------------------------------------------------------------- tile order
// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8).  Each XCD gets one contiguous range of the linear tile order, and in
// that order tiles come in groups of group_m m-tiles x all n-tiles with m
// fastest, so the workgroups resident on one XCD at a time share A and B
// slabs in that XCD's L2.  k-splits are outermost.
struct TileCoord {
  int tm, tn, split;
  bool valid;
};

__device__ inline TileCoord tile_coord(const GemmParams& p) {
  const int per_split = p.tiles_m * p.tiles_n;
  const int total = per_split * p.splits;
  const int per_xcd = (total + 7) / 8;
  const int b = blockIdx.x;
  const int lin = (b & 7) * per_xcd + (b >> 3);
  TileCoord tc;
  tc.valid = lin < total;
  const int l = tc.valid ? lin : 0;
  tc.split = l / per_split;
  const int t = l - tc.split * per_split;
  const int gsz = p.group_m * p.tiles_n;
  const int grp = t / gsz;
  const int first_m = grp * p.group_m;
  const int width = min(p.tiles_m - first_m, p.group_m);
  const int r = t - grp * gsz;
  tc.tm = first_m + r % width;
  tc.tn = r / width;
  return tc;
}

// ---------------------------------------------------------------- the kernel
template <typename T, int BM, int BN, int WM, int WN, bool AK, bool BKM, int EPI>
__global__ void __launch_bounds__(WM* WN * 64) gemm_kernel(GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = ElemTraits<T>::kBK;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int SUB = BK / 16;
  typedef TileLayout<T, BM, AK> LA;
  typedef TileLayout<T, BN, BKM> LB;
  typedef TileLoader<T, BM, NT, AK> GA;
  typedef TileLoader<T, BN, NT, BKM> GB;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(EPI != EPI_LOGITS || WTM == 128, "logit partials are per 128-row slice");
  constexpr int STAGE = LA::kBytes + LB::kBytes;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const TileCoord tc = tile_coord(p);
  if (!tc.valid) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int kt_begin = tc.split * p.k_tiles_per_split;
  const int kt_end = min(p.k_tiles, kt_begin + p.k_tiles_per_split);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[GA::kNCH], rb[GB::kNCH];
  GA::load(ra, p.a, m0, (int64_t)kt_begin * BK, tid);
  GB::load(rb, p.b, n0, (int64_t)kt_begin * BK, tid);
  GA::store(smem, ra, tid);
  GB::store(smem + LA::kBytes, rb, tid);
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int cur = (kt - kt_begin) & 1;
    const bool more = kt + 1 < kt_end;
    if (more) {
      GA::load(ra, p.a, m0, (int64_t)(kt + 1) * BK, tid);
      GB::load(rb, p.b, n0, (int64_t)(kt + 1) * BK, tid);
    }
    const char* sa = smem + cur * STAGE;
    const char* sb = sa + LA::kBytes;
#pragma unroll
    for (int kk = 0; kk < SUB; ++kk) {
      typename Frag<T>::type fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = load_frag<T, BM, AK>(sa, wm * WTM + i * 32, kk, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = load_frag<T, BN, BKM>(sb, wn * WTN + j * 32, kk, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_block(fa[i], fb[j], acc[i][j]);
    }
    if (more) {
      char* nxt = smem + (cur ^ 1) * STAGE;
      GA::store(nxt, ra, tid);
      GB::store(nxt + LA::kBytes, rb, tid);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogues
  const int h = lane >> 5, col = lane & 31;
  if constexpr (EPI == EPI_LOGITS) {
    // D rows are vocabulary ids (m), columns are tokens (n).  Per token this
    // lane holds 64 of the 128 logits of its wave's slice; its partner lane
    // (lane ^ 32) holds the other 64.
    const int64_t mw = m0 + wm * WTM;
    const int slice = (int)(mw / 128);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn * WTN + j * 32 + col;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = mw + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
          if (m < p.valid_m) mx = fmaxf(mx, acc[i][j][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = mw + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
          if (m < p.valid_m) s += __expf(acc[i][j][r] - mx);
        }
      s += __shfl_xor(s, 32);
      const bool nvalid = n < p.valid_n;
      if (h == 0 && nvalid && slice < p.n_slices) p.part[n * p.n_slices + slice] = make_float2(mx, s);
      if (nvalid) {
        float* zrow = p.out + n * p.ldo;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t m = mw + i * 32 + q * 8 + h * 4;
            f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            if (m + 3 < p.valid_m) {
              *(f32x4*)(zrow + m) = v;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (m + e < p.valid_m) zrow[m + e] = v[e];
            }
          }
      }
    }
  } else {
    float* out = p.out + (EPI == EPI_SLAB ? (int64_t)tc.split * p.split_stride : 0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + wn * WTN + j * 32 + col;
        if (n >= p.valid_n) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
          if (m < p.valid_m) {
            float* dst = out + m * p.ldo + n;
            if (EPI == EPI_ACCUM && p.beta)
              *dst += acc[i][j][r];
            else
              *dst = acc[i][j][r];
          }
        }
      }
  }
}

}  // namespace ckl
