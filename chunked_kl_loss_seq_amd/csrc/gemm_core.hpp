// MFMA GEMM engine for gfx950 (CDNA4), shared by the three contractions of the
// fused chunked KL loss:
//   logits    Z^T tile = W . H_c^T   (both operands contiguous along d)
//   dH        dH_c     = G . W       (G contiguous along V, W contiguous along d)
//   dW        dW      += G^T . H_c   (both operands contiguous along the token axis)
//
// One workgroup computes a BM x BN tile of D = A . B with WM x WN waves.  The
// reduction runs over k-slabs of BK = KB / sizeof(T) elements, copied global ->
// LDS by buffer_load ... lds into a ring of NS stages, so NS - 1 slabs are in
// flight while one is consumed:
//   * an operand contiguous along k ("k-major") is kept as [row][KB bytes]
//     with a 16-byte-chunk XOR swizzle and read as one ds_read_b128 per MFMA
//     fragment;
//   * an operand contiguous along m or n ("mn-major") is kept as it lies in
//     memory, [k][row], with a 64-byte-block XOR swizzle, and read with
//     ds_read_tr16_b64, which hands each lane four k-consecutive 16-bit values
//     of one column (two reads per bf16 fragment).  fp32 mn-major operands use
//     ds_read_b32.
// bf16 operands use v_mfma_f32_32x32x16_bf16 (MS = 32), or for two k-major
// operands v_mfma_f32_16x16x32_bf16 (MS = 16: the same flops in 16 x 16
// blocks, which sustain a higher rate under the board's power limit); fp32
// operands use v_mfma_f32_32x32x2_f32 over the same LDS layout.  A 32-row
// fragment holds the 8 k-values k0 + 8h .. k0 + 8h + 7 of lane half h, a
// 16-row one k0 + 8q .. k0 + 8q + 7 of lane quarter q; the fp32 path issues 8
// MFMAs, one per element, which pair the same k on the A and B side.
//
// Accumulator layouts (checked on gfx950): in a 32x32 block lane l, slot r
// holds D[(r/4)*8 + (l/32)*4 + r%4][l%32]; in a 16x16 block lane l, slot r
// holds D[(l/16)*4 + r][l%16].
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

// One GEMM operand in global memory, stored as rows of a row-major matrix:
// a k-major operand has storage row = mn and column = k, an mn-major one
// storage row = k and column = mn.  Element (row, col) lives at
//   ptr[row * ld + col]                                        (blk == 0), or
//   ptr[(row / 64) * blk + (col / 64) * 4096 + (row % 64) * 64 + col % 64]
// in the tiled layout of 64 x 64 element tiles (blk = elements between two
// tile rows).  Rows mn >= mn_ext and columns k >= k_ext read as zero.
struct Operand {
  const void* ptr;
  int64_t ld;
  int64_t mn_ext;
  int64_t k_ext;
  int64_t blk;
};

__device__ inline int64_t elem_offset(const Operand& o, int64_t row, int64_t col) {
  if (o.blk == 0) return row * o.ld + col;
  return (row >> 6) * o.blk + (col >> 6) * 4096 + (row & 63) * 64 + (col & 63);
}

constexpr float kLog2e = 1.4426950408889634f;

// exp(z - mx) for the logits epilogue, nmx = -mx log2(e).  Values kept in
// bf16 take 2^(z log2(e) + nmx), one fma and one exp instruction: its error,
// |mx| log2(e) 2^-24 in the exponent, is far below bf16 rounding.  fp32
// values take the subtraction first, exact for z near mx.
template <typename T>
__device__ inline float slice_exp(float z, float mx, float nmx) {
  if constexpr (sizeof(T) == 2) return __builtin_amdgcn_exp2f(__builtin_fmaf(z, kLog2e, nmx));
  return __expf(z - mx);
}

enum EpilogueKind : int {
  EPI_LOGITS = 0,  // per (n, 128-row slice of m): mx = max D, P[n][m] = exp(D[m][n] - mx), (mx, sum P)
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
  void* out;             // EPI_LOGITS: exp values (tiled, element type T); else fp32 slab base or dW
  int64_t ldo;           // EPI_LOGITS: elements between tile rows of out; else row stride
  int64_t split_stride;  // elements between k-split slabs (EPI_SLAB)
  int64_t valid_m, valid_n;  // stores are limited to m < valid_m, n < valid_n
  float2* part;          // EPI_LOGITS: partial (max, sum exp) per [n][slice]
  int n_slices;          // EPI_LOGITS: slices per row of part
  int beta;              // EPI_ACCUM
  // Device int or null: the chunk's rows (tokens) at and after *live are all
  // masked.  Logits tiles of those rows return at once, dH tiles of them
  // write zeros without a k-loop, and dW (k = rows) stops its k-loop there.
  const int* live;
  // EPI_LOGITS, or null: the cached ids of the chunk's rows by 256-id
  // vocabulary tile p (slices 2p, 2p + 1): 128-bit masks id_bits[p][n][h] of
  // slice 2p + h, and two uint16 id_pre[p][n] of the row's distinct cached ids
  // below each slice (row stride id_cpad).  The fp32 logit at every masked
  // (id, n) is copied out of the accumulators, before they become exp values,
  // to zs[n * zk + rank], rank = the count below the slice + the mask bits
  // below the id.
  const void* id_bits;
  const void* id_pre;
  int64_t id_cpad;
  float* zs;
  int zk;
  // EPI_LOGITS, or null: the rows' log-normalisers are already known (the
  // recomputing backward), so the epilogue stores the gradient's dense part
  // G = f p, f = w exp(mx - lse), itself, with the same fp32 operations as the
  // separate dense pass: lse of row n is g_lse[g_rowmap ? g_rowmap[n] : n];
  // w = *g_scale (times *g_gscale if not null) for rows below valid_n (and
  // *live), 0 for the others; ids at or past valid_m get 0.
  const float* g_lse;
  const int* g_rowmap;
  const float* g_scale;
  const float* g_gscale;
};

// ---------------------------------------------------------------- LDS layouts
// One wave instruction of buffer_load ... lds moves 1 KiB, lane l's 16 bytes
// landing at byte 16 l of that KiB, so the LDS layouts are fixed by which
// global chunk each lane fetches.  The swizzles keep the fragment reads free of
// bank conflicts on gfx950's 64-bank (256 bytes per clock) LDS, which serves a
// ds_read_b128 16 lanes at a time and a ds_read_b64 32 lanes at a time.
//
// k-major slab: [R rows][KB bytes]; the 16-byte chunk c of row r sits at
// chunk c ^ ((r / (256 / KB)) % (KB / 16)): the 16 rows one fragment read
// serves together fall on 16 distinct 16-byte bank groups.
template <int R, int KB>
struct KTile {
  static constexpr int kCPR = KB / 16;          // chunks per row
  static constexpr int kRowsPerBankRow = 256 / KB;
  static constexpr int kBytes = R * KB;
  __device__ static inline int off(int row, int chunk) {
    return row * KB + ((chunk ^ ((row / kRowsPerBankRow) % kCPR)) << 4);
  }
};

// mn-major slab: [BK k-rows][R * sizeof(T) bytes]; the 64-byte block j of
// k-row k sits at block j ^ swz(k).  A ds_read_tr16_b64 serves 32 lanes that
// read the same 64-byte block of 4 consecutive k-rows; swz puts those four
// blocks in the four distinct 64-byte bank quarters.
template <typename T, int R, int BK>
struct MNTile {
  static constexpr int kRowBytes = R * (int)sizeof(T);
  static constexpr int kBytes = BK * kRowBytes;
  static constexpr int kStep = (kRowBytes / 64) % 4;  // bank quarter advance per k-row
  static_assert(kRowBytes % 256 == 0 || kRowBytes % 256 == 128, "unsupported mn-major tile width");
  __device__ static inline int swz(int k) { return kStep == 0 ? (k & 3) : ((k >> 1) & 1); }
  // byte address of logical byte lb (= column * sizeof(T)) of k-row k
  __device__ static inline int off(int k, int lb) { return k * kRowBytes + ((((lb >> 6) ^ swz(k)) << 6) | (lb & 63)); }
};

// ---------------------------------------------------------------- global -> LDS
// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt split over bits 3:0 and 15:14;
// expcnt and lgkmcnt left at their "no wait" maxima).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past the range: the load returns zeros

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + 2 GiB) with raw (unswizzled) addressing.
// The base is wave-uniform; readfirstlane makes that explicit so the resource
// lives in SGPRs.
__device__ inline i32x4 make_rsrc(const void* base) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r.x = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  r.y = (int32_t)(__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xFFFFu);  // stride 0
  r.z = 0x7FFFFFF0;                                                                 // num_records (bytes)
  r.w = 0x00020000;                                                                 // raw buffer, 32-bit data format
  return r;
}

// A 64-bit value the caller knows to be wave-uniform, kept in SGPRs.
__device__ inline uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// buffer_load_dwordx4 ... lds: lane l's 16 bytes at byte `voff` of the
// resource go to LDS byte lds_addr + 16 l (lds_addr is wave-uniform and goes
// through M0).  Written as inline assembly so that the compiler's wait-count
// pass, which cannot tell these LDS writes apart from the fragment reads of
// other stages, does not put a full vmcnt wait in front of every LDS read;
// the kernel orders them itself with explicit vmcnt waits and barriers.  The
// instruction has no destination VGPRs.  On GFX9 an LDS DMA must not follow a
// scalar write of M0 directly (one wait state), hence the s_nop.
__device__ inline void dma16(const i32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(lds_addr)
               : "memory", "m0");
}

__device__ inline uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p);
}

// Per-lane state to copy one operand's k-slabs of a tile into LDS.  Lane
// offsets are relative to the slab origin and do not change along k; rows
// past mn_ext are folded in as out-of-range offsets, k past k_ext is checked
// on the last slabs only.  The slab's 1 KiB blocks are dealt to the waves in
// turn; when they do not divide evenly, a wave short of a block issues an
// out-of-range load into a spare 1 KiB of LDS instead, so that every wave has
// the same number of loads in flight per slab.
template <typename T, int R, int NW, bool KMAJ, int KB>
struct SlabDMA {
  static constexpr int kEPC = 16 / (int)sizeof(T);
  static constexpr int kBK = KB / (int)sizeof(T);
  static constexpr int kBytes = KMAJ ? KTile<R, KB>::kBytes : MNTile<T, R, kBK>::kBytes;
  static constexpr int kBlocks = kBytes / 1024;
  static constexpr int kNI = (kBlocks + NW - 1) / NW;  // load instructions per wave per slab (at most)
  static constexpr bool kEven = kBlocks % NW == 0;
  static_assert(kBytes % 1024 == 0, "slab must be whole KiB blocks");

  uint32_t voff[kNI];

  // k offset of this lane's chunk i within the slab (recomputed on tail slabs,
  // so that it holds no registers through the main loop)
  __device__ static inline int kdel(int wave, int lane, int i) {
    const int q = (i * NW + wave) * 1024 + lane * 16;
    if (KMAJ) {
      typedef KTile<R, KB> L;
      const int row = q / KB;
      const int pc = (q % KB) >> 4;
      return (pc ^ ((row / L::kRowsPerBankRow) % L::kCPR)) * kEPC;
    }
    return q / MNTile<T, R, kBK>::kRowBytes;
  }

  __device__ static inline bool has(int wave, int i) { return kEven || i * NW + wave < kBlocks; }
  static constexpr int kSpare = kEven ? 0 : 1024;  // LDS bytes for the padding loads

  // Lane offsets relative to the slab origin.  The origin (row0, col0) of
  // every slab of a tile has row0 and col0 aligned to the tile (64 elements)
  // along mn and to the slab depth along k, and a slab never crosses a
  // 64-element tile boundary along k, so these offsets are the same for all
  // slabs of the tile in both layouts.
  __device__ inline void init(const Operand& o, int64_t mn0, int wave, int lane) {
    // representative origin: k0 = 0
    const int64_t r0 = KMAJ ? mn0 : 0, c0 = KMAJ ? 0 : mn0;
    const int64_t base = elem_offset(o, r0, c0);
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      const int b = i * NW + wave;
      int row_mn, kd;
      int64_t e;
      if (KMAJ) {
        typedef KTile<R, KB> L;
        const int q = b * 1024 + lane * 16;
        const int row = q / KB;
        const int pc = (q % KB) >> 4;
        const int c = pc ^ ((row / L::kRowsPerBankRow) % L::kCPR);
        row_mn = row;
        kd = c * kEPC;
        e = elem_offset(o, r0 + row, c0 + kd) - base;
      } else {
        typedef MNTile<T, R, kBK> L;
        const int q = b * 1024 + lane * 16;
        const int krow = q / L::kRowBytes;
        const int pb = q % L::kRowBytes;
        const int lb = (((pb >> 6) ^ L::swz(krow)) << 6) | (pb & 63);
        row_mn = lb / (int)sizeof(T);
        kd = krow;
        e = elem_offset(o, r0 + kd, c0 + row_mn) - base;
      }
      voff[i] = (uint32_t)(e * (int64_t)sizeof(T));
      if (mn0 + row_mn >= o.mn_ext) voff[i] = kOOB;
    }
  }

  // Element offset of the slab at depth k0 from the slab at depth 0 (same
  // tile origin).  It depends on k0 and the layout only, so a tile keeps one
  // base address and advances it per slab with scalar arithmetic.
  __device__ static inline int64_t slab_off(const Operand& o, int64_t k0) {
    if (KMAJ) return o.blk ? (k0 >> 6) * 4096 + (k0 & 63) : k0;
    return o.blk ? (k0 >> 6) * o.blk + (k0 & 63) * 64 : k0 * o.ld;
  }

  // Issue the copy of a whole slab (every k inside the operand) whose origin
  // is at byte address `base` into this wave's blocks of the stage at LDS byte
  // address `lds` (wave-uniform; blocks of other waves are 1 KiB apart).
  __device__ inline void issue_full(uint64_t base, uint32_t lds, int wave, uint32_t spare) const {
    const i32x4 rs = make_rsrc((const void*)base);
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      const bool real = has(wave, i);
      dma16(rs, real ? voff[i] : kOOB, real ? lds + (uint32_t)((i * NW + wave) * 1024) : spare);
    }
  }

  // Same for a slab that reaches past k_ext: only the first kleft k (none when
  // kleft <= 0) are loaded, the rest read as zeros without touching memory.
  __device__ inline void issue_tail(uint64_t base, uint32_t lds, int wave, int lane, uint32_t spare,
                                    int kleft) const {
    const i32x4 rs = make_rsrc((const void*)base);
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      const bool real = has(wave, i);
      const uint32_t v = (!real || kdel(wave, lane, i) >= kleft) ? kOOB : voff[i];
      dma16(rs, v, real ? lds + (uint32_t)((i * NW + wave) * 1024) : spare);
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

// Fragment of 32 rows (row0 .. row0+31 of the tile) x 16 k (sub-step kk):
// lane l gets row row0 + l % 32, k = 16 kk + 8 (l / 32) .. + 7.
template <typename T, int R, bool KMAJ, int KB>
__device__ inline typename Frag<T>::type load_frag(const char* lds, int row0, int kk, int lane) {
  const int h = lane >> 5;
  if constexpr (KMAJ) {
    typedef KTile<R, KB> L;
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
    typedef MNTile<T, R, KB / (int)sizeof(T)> L;
    if constexpr (sizeof(T) == 2) {
      // 16-lane group g: columns (g & 1) * 16 .., k block (g >> 1) * 8.
      // Within the group, source lane 4j + p reads k-row j (+4 for the second
      // read) at columns 4p .. 4p+3; the transpose hands lane i column i.
      const int g = lane >> 4, i = lane & 15;
      const int krow = 16 * kk + (g >> 1) * 8 + (i >> 2);
      const int lb = (row0 + (g & 1) * 16 + 4 * (i & 3)) * 2;
      const char* p0 = lds + L::off(krow, lb);
      const char* p1 = lds + L::off(krow + 4, lb);
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
      const int lb = (row0 + (lane & 31)) * 4;
      f32x8 f;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = *(const float*)(lds + L::off(16 * kk + 8 * h + j, lb));
      return f;
    }
  }
}

// bf16 fragment of 16 rows (row0 .. row0+15) x 32 k (sub-step kk) of a
// k-major slab for v_mfma_f32_16x16x32_bf16: lane l gets row row0 + l % 16,
// k = 32 kk + 8 (l / 16) .. + 7.  The 16 lanes one ds_read_b128 serves together
// read 16 consecutive rows at one chunk, as in the 32-row fragments.
template <int R, int KB>
__device__ inline bf16x8 load_frag16(const char* lds, int row0, int kk, int lane) {
  typedef KTile<R, KB> L;
  const u32x4 v = *(const u32x4*)(lds + L::off(row0 + (lane & 15), 4 * kk + (lane >> 4)));
  return __builtin_bit_cast(bf16x8, v);
}

__device__ inline f32x4 mfma_block(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// ---------------------------------------------------------------- cached-id logits
// Slot r (0..3 or 0..15, varying per lane) of an accumulator block, by selects
// on constant slots: a register index that differs between lanes would
// otherwise go through scratch memory.
__device__ inline float pick4(const f32x4& v, int r) {
  const float a = (r & 1) ? v[1] : v[0];
  const float b = (r & 1) ? v[3] : v[2];
  return (r & 2) ? b : a;
}
__device__ inline float pick16(const f32x16& v, int r) {
  float q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = (r & 1) ? v[4 * i + 1] : v[4 * i];
    const float b = (r & 1) ? v[4 * i + 3] : v[4 * i + 2];
    q[i] = (r & 2) ? b : a;
  }
  const float lo = (r & 4) ? q[1] : q[0];
  const float hi = (r & 4) ? q[3] : q[2];
  return (r & 8) ? hi : lo;
}

// Gradient weight of the recomputing backward (EPI_LOGITS with g_lse): w and
// the compacted chunk's row count (all rows when not compacted).
__device__ inline void grad_weight(const GemmParams& p, float& w, int& live) {
  w = p.g_gscale != nullptr ? *p.g_scale * *p.g_gscale : *p.g_scale;
  live = p.live != nullptr ? __builtin_amdgcn_readfirstlane(*p.live) : 0x7FFFFFFF;
}
// Whether token n is a row of the chunk (of its compacted rows): rows past it
// hold no exp values, possibly not even numbers, and are stored as zeros.
__device__ inline bool grad_row(const GemmParams& p, int64_t n, int live) { return n < p.valid_n && n < live; }
// f = w exp(mx - lse) of row n's slice: the factor the dense pass would apply.
__device__ inline float grad_factor(const GemmParams& p, int64_t n, float mx, float w, int live) {
  if (!grad_row(p, n, live)) return 0.f;
  const float lse = p.g_lse[p.g_rowmap != nullptr ? p.g_rowmap[n] : n];
  return w * __expf(mx - lse);
}

// LDS bytes after the stage ring for the tile's id tables: 256 tokens x 2
// slices x 16-byte masks, then 256 tokens x (count below slice s0, count below
// slice s0 + 1) as two uint16.
constexpr int kIdBitsBytes = 256 * 32;
constexpr int kIdTabBytes = kIdBitsBytes + 256 * 4;

// ---------------------------------------------------------------- the kernel
template <int MS>
struct AccOf {
  typedef f32x16 type;  // 32 x 32 block
};
template <>
struct AccOf<16> {
  typedef f32x4 type;  // 16 x 16 block
};

// At most 256 VGPRs per lane (two waves per SIMD), so that either one 8-wave
// or two 4-wave workgroups fit a compute unit; with two workgroups their
// barriers and epilogues overlap each other's MFMA work.  MS is the MFMA
// block (32, or 16 for bf16 with both operands k-major).
template <typename T, int BM, int BN, int WM, int WN, bool AK, bool BKM, int EPI, int KB, int NS, int MS = 32>
__global__ void __launch_bounds__(WM* WN * 64) __attribute__((amdgpu_waves_per_eu(2))) gemm_kernel(GemmParams p) {
  constexpr int NW = WM * WN;
  constexpr int BK = KB / (int)sizeof(T);
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / MS, FN = WTN / MS;
  constexpr int SUB = BK / (MS == 32 ? 16 : 32);
  constexpr int NR = MS == 32 ? 16 : 4;  // accumulator slots per block
  constexpr int NMF = FM * FN;
  typedef SlabDMA<T, BM, NW, AK, KB> DA;
  typedef SlabDMA<T, BN, NW, BKM, KB> DB;
  constexpr int NIT = DA::kNI + DB::kNI;  // this wave's loads per slab
  static_assert(MS == 32 || (MS == 16 && sizeof(T) == 2 && AK && BKM && EPI == EPI_LOGITS),
                "16 x 16 blocks: bf16 logits (both operands k-major) only");
  static_assert(WTM % MS == 0 && WTN % MS == 0, "wave tile must be a multiple of the MFMA block");
  static_assert(SUB % 2 == 0 && SUB >= 2, "the pipeline assumes an even sub-step count");
  static_assert(NS >= 2 && (NS - 1) * NIT < 64, "stages in flight must fit the vmcnt counter");
  static_assert(EPI != EPI_LOGITS || WTM == 128, "logit partials are per 128-row slice");
  constexpr int STAGE = DA::kBytes + DB::kBytes;
  constexpr int SPARE = DA::kSpare > DB::kSpare ? DA::kSpare : DB::kSpare;
  constexpr int XOFF = NS * STAGE + SPARE;  // id tables (logits only)
  constexpr int XBYTES = EPI == EPI_LOGITS ? kIdTabBytes : 0;
  static_assert(EPI != EPI_LOGITS || (BN == 256 && BM == 256 && NW == 8 && WM == 2), "id tables: 256 x 256 tiles");
  __shared__ __attribute__((aligned(1024))) char smem[XOFF + XBYTES];
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t spare = lds0 + NS * STAGE;

  const TileCoord tc = tile_coord(p);
  if (!tc.valid) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int64_t m0 = (int64_t)tc.tm * BM, n0 = (int64_t)tc.tn * BN;
  const int kt_begin = tc.split * p.k_tiles_per_split;
  int kt_end = min(p.k_tiles, kt_begin + p.k_tiles_per_split);
  if (p.live != nullptr) {
    const int lv = __builtin_amdgcn_readfirstlane(*p.live);
    if constexpr (EPI == EPI_LOGITS) {
      if (n0 >= lv) return;  // whole workgroup: no barrier reached yet
    } else if constexpr (EPI == EPI_SLAB) {
      if (m0 >= lv) kt_end = kt_begin;  // the epilogue writes this tile's zeros
    } else {
      kt_end = min(kt_end, (lv + BK - 1) / BK);  // rows are the k dimension
    }
  }

  typename AccOf<MS>::type acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[i][j][r] = 0.f;

  typedef typename Frag<T>::type FragT;
  FragT fa[2][FM], fb[2][FN];
  auto lfa = [&](const char* base, int i, int kk, int ln) -> FragT {
    if constexpr (MS == 16) return load_frag16<BM, KB>(base, wm * WTM + i * 16, kk, ln);
    else return load_frag<T, BM, AK, KB>(base, wm * WTM + i * 32, kk, ln);
  };
  auto lfb = [&](const char* base, int j, int kk, int ln) -> FragT {
    if constexpr (MS == 16) return load_frag16<BN, KB>(base, wn * WTN + j * 16, kk, ln);
    else return load_frag<T, BN, BKM, KB>(base, wn * WTN + j * 32, kk, ln);
  };
  DA da;
  DB db;
  da.init(p.a, m0, wave, lane);
  db.init(p.b, n0, wave, lane);
  // byte addresses of the tile's slab origins at k = 0 (wave-uniform)
  const uint64_t a_org = uniform64((uint64_t)p.a.ptr + sizeof(T) * (uint64_t)(AK ? elem_offset(p.a, m0, 0)
                                                                               : elem_offset(p.a, 0, m0)));
  const uint64_t b_org = uniform64((uint64_t)p.b.ptr + sizeof(T) * (uint64_t)(BKM ? elem_offset(p.b, n0, 0)
                                                                                : elem_offset(p.b, 0, n0)));

  // Copy slab kt into stage st.  A slab past the tile's k range is skipped
  // when skip is set (the waits then count fewer loads, which only the
  // two-stage ring, whose waits drain everything, tolerates), otherwise it
  // is issued as out-of-range loads so every wave keeps NIT loads per slab.
  auto issue = [&](int kt, int st, bool skip) {
    const int64_t k0 = (int64_t)kt * BK;
    const uint32_t sa_lds = lds0 + (uint32_t)(st * STAGE), sb_lds = sa_lds + DA::kBytes;
    if (kt < kt_end && k0 + BK <= p.a.k_ext) {
      da.issue_full(a_org + sizeof(T) * (uint64_t)DA::slab_off(p.a, k0), sa_lds, wave, spare);
      db.issue_full(b_org + sizeof(T) * (uint64_t)DB::slab_off(p.b, k0), sb_lds, wave, spare);
    } else if (kt < kt_end || !skip) {
      const int kleft = kt < kt_end ? (int)(p.a.k_ext - k0) : 0;
      da.issue_tail(kt < kt_end ? a_org + sizeof(T) * (uint64_t)DA::slab_off(p.a, k0) : a_org, sa_lds, wave, lane, spare,
                    kleft);
      db.issue_tail(kt < kt_end ? b_org + sizeof(T) * (uint64_t)DB::slab_off(p.b, k0) : b_org, sb_lds, wave, lane, spare,
                    kleft);
    }
  };

  // The logits tile's id tables (8 KiB of masks and 1 KiB of count pairs, both
  // contiguous) go to LDS ahead of the first slabs, so the prologue's wait
  // covers them: wave w copies the masks of tokens 32 w .. 32 w + 31 (lane l:
  // token 32 w + l / 2, slice 2 tm + l % 2), wave 0 also the count pairs.
  // Masks of tokens past valid_n and of a slice past the vocabulary read as
  // zeros; count pairs are only read where a mask bit is set.
  if constexpr (EPI == EPI_LOGITS) {
    if (p.id_bits != nullptr) {
      const uint64_t bbase = uniform64((uint64_t)p.id_bits + ((uint64_t)tc.tm * p.id_cpad + n0) * 32);
      const int t = 32 * wave + (lane >> 1), sl = lane & 1;
      const bool ok = n0 + t < p.valid_n && 2 * tc.tm + sl < p.n_slices;
      dma16(make_rsrc((const void*)bbase), ok ? (uint32_t)(wave * 1024 + lane * 16) : kOOB,
            lds0 + XOFF + (uint32_t)wave * 1024u);
      if (wave == 0) {
        const uint64_t pbase = uniform64((uint64_t)p.id_pre + ((uint64_t)tc.tm * p.id_cpad + n0) * 4);
        dma16(make_rsrc((const void*)pbase), (uint32_t)(lane * 16), lds0 + XOFF + kIdBitsBytes);
      }
    }
  }

  // Ring of NS LDS stages.  At the top of iteration kt the stage cur holds
  // slab kt and the other stages hold (or are loading) slabs kt+1 .. kt+NS-1.
  // In the last sub-step of iteration kt each wave waits for its part of slab
  // kt+1, the workgroup synchronises half-way through the MFMAs, the first
  // fragments of slab kt+1 load, slab kt+NS is issued into stage cur (no wave
  // reads it any more), and the second half of the MFMAs runs.  The loop is
  // unrolled over the NS stages so that every LDS address is a constant offset
  // from a per-lane base.
#pragma unroll
  for (int st = 0; st < NS; ++st) issue(kt_begin + st, st, false);
  wait_vmcnt<(NS - 1) * NIT>();
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FM; ++i) fa[0][i] = lfa(smem, i, 0, lane);
#pragma unroll
  for (int j = 0; j < FN; ++j) fb[0][j] = lfb(smem + DA::kBytes, j, 0, lane);

  for (int kt0 = kt_begin; kt0 < kt_end; kt0 += NS) {
#pragma unroll
    for (int cur = 0; cur < NS; ++cur) {
      const int kt = kt0 + cur;
      if (kt >= kt_end) break;
      const int nxt = cur + 1 == NS ? 0 : cur + 1;
      const char* sa = smem + cur * STAGE;
      const char* sb = sa + DA::kBytes;
      const char* na = smem + nxt * STAGE;
      const char* nb = na + DA::kBytes;
#pragma unroll
      for (int kk = 0; kk < SUB; ++kk) {
        const int fbuf = kk & 1;
        // With 32 blocks per sub-step the fragment addresses are recomputed
        // in each sub-step: hoisted out of the loop they would not fit the
        // register budget.
        int ln = lane;
        if constexpr (NMF > 8) asm volatile("" : "+v"(ln));
        if (kk + 1 < SUB) {
#pragma unroll
          for (int i = 0; i < FM; ++i) fa[fbuf ^ 1][i] = lfa(sa, i, kk + 1, ln);
#pragma unroll
          for (int j = 0; j < FN; ++j) fb[fbuf ^ 1][j] = lfb(sb, j, kk + 1, ln);
#pragma unroll
          for (int q = 0; q < NMF; ++q)
            acc[q / FN][q % FN] = mfma_block(fa[fbuf][q / FN], fb[fbuf][q % FN], acc[q / FN][q % FN]);
          if constexpr (MS == 16) {
            // one fragment read every two MFMAs (measured faster than the
            // scheduler's own order for this loop)
#pragma unroll
            for (int q = 0; q < FM + FN; ++q) {
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NMF - 2 * (FM + FN), 0);
          }
          if constexpr (!AK && !BKM) {
            // both operands come through transpose reads (two per fragment):
            // pin one MFMA, two LDS reads, ... (measured faster for this shape)
#pragma unroll
            for (int q = 0; q < NMF; ++q) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < NMF / 2; ++q)
            acc[q / FN][q % FN] = mfma_block(fa[fbuf][q / FN], fb[fbuf][q % FN], acc[q / FN][q % FN]);
          wait_vmcnt<(NS - 2) * NIT>();
          __syncthreads();
#pragma unroll
          for (int i = 0; i < FM; ++i) fa[0][i] = lfa(na, i, 0, ln);
#pragma unroll
          for (int j = 0; j < FN; ++j) fb[0][j] = lfb(nb, j, 0, ln);
          issue(kt + NS, cur, NS == 2);
#pragma unroll
          for (int q = NMF / 2; q < NMF; ++q)
            acc[q / FN][q % FN] = mfma_block(fa[fbuf][q / FN], fb[fbuf][q % FN], acc[q / FN][q % FN]);
        }
      }
    }
  }
  wait_vmcnt<0>();  // no LDS copy outlives the workgroup

  // ------------------------------------------------------------ epilogues
  // Lane l, accumulator slot r of block (i, j) holds D[row][col] with
  // row = mw + 32 i + 8 (r / 4) + 4 (l / 32) + r % 4 and col = nw + 32 j + l % 32.
  const int h = lane >> 5, col = lane & 31;
  const int64_t mw = m0 + wm * WTM, nw = n0 + wn * WTN;
  const bool full = (mw + WTM <= p.valid_m) && (nw + WTN <= p.valid_n);
  if constexpr (MS == 16) {
    // Logits from 16 x 16 blocks: lane l, slot r of block (i, j) holds the
    // logit of id mw + 16 i + 4 g + r (g = l / 16) and token nw + 16 j + c
    // (c = l % 16), so the four lanes c, c + 16, c + 32, c + 48 hold a token's
    // 128 slice logits, 32 each.  Same outputs as the 32-wide epilogue below.
    static_assert(WTM == 128 && WTN == 64 && NW * 16384 <= NS * STAGE, "one wave = two 64 x 64 tiles");
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
    const int g = lane >> 4, c = lane & 15;
    const int slice = (int)(mw / 128);
    const bool mfull = mw + WTM <= p.valid_m;
    const int m0lane = (int)mw + 4 * g;
    const int vm = (int)(p.valid_m < (int64_t)0x7FFFFFFF ? p.valid_m : (int64_t)0x7FFFFFFF);
    // the cached-id masks of this lane's FN tokens in the wave's slice, all
    // read before the first is needed (one LDS round trip)
    u32x4 idw[FN];
    uint32_t idpre[FN];
    float gf[FN];
    float gw = 0.f;
    int glive = 0x7FFFFFFF;
    if (p.g_lse != nullptr) grad_weight(p, gw, glive);
    if (p.id_bits != nullptr) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int t = (int)(nw - n0) + 16 * j + c;
        idw[j] = *(const u32x4*)(smem + XOFF + t * 32 + wm * 16);
        idpre[j] = *(const uint32_t*)(smem + XOFF + kIdBitsBytes + 4 * t);
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = nw + 16 * j + c;
      if (p.id_bits != nullptr) {
        // logits at the cached ids of token n in this wave's slice: lane
        // quarter g holds bits 4 g .. 4 g + 3 of every 16 (block i = bit / 16,
        // slot = bit % 4)
        const u32x4 w = idw[j];
        const uint32_t lm = 0x000F000Fu << (4 * g);
        if (((w.x | w.y | w.z | w.w) & lm) != 0u) {
          uint32_t run = (idpre[j] >> (16 * wm)) & 0xFFFFu;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t word = w[q];
            uint32_t m = word & lm;
            while (m != 0u) {
              const int b = __builtin_ctz(m);
              m &= m - 1u;
              const uint32_t rk = run + (uint32_t)__builtin_popcount(word & ((1u << b) - 1u));
              const float lo = pick4(acc[2 * q][j], b & 3), hi = pick4(acc[2 * q + 1][j], b & 3);
              if (rk < (uint32_t)p.zk) p.zs[n * p.zk + rk] = (b & 16) ? hi : lo;
            }
            run += (uint32_t)__builtin_popcount(word);
          }
        }
      }
      float mx = -INFINITY, sum = 0.f;
      if (mfull) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, acc[i][j][r]);
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, m0lane + 16 * i + r < vm ? acc[i][j][r] : -INFINITY);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float nmx = -mx * kLog2e;
      if (mfull) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = slice_exp<T>(acc[i][j][r], mx, nmx);
            acc[i][j][r] = e;
            sum += e;
          }
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = slice_exp<T>(acc[i][j][r], mx, nmx);
            acc[i][j][r] = e;
            sum += m0lane + 16 * i + r < vm ? e : 0.f;
          }
      }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      if (g == 0 && n < p.valid_n && slice < p.n_slices) p.part[n * p.n_slices + slice] = make_float2(mx, sum);
      if (p.g_lse != nullptr) {
        gf[j] = grad_factor(p, n, mx, gw, glive);
        if (!grad_row(p, n, glive)) {
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;  // f = 0 then stores zeros
        }
      }
    }
    // The exp values (or, with g_lse, the gradient values) leave through this
    // wave's 16 KiB of LDS in the tiles' own order (token row t of tile i / 4,
    // 16-byte chunks XOR-swizzled by the row) as 16 coalesced 1 KiB stores, as
    // in the 32-wide epilogue.
    if (p.g_lse != nullptr) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][r] = (mfull || m0lane + 16 * i + r < vm) ? gf[j] * (float)(__bf16)acc[i][j][r] : 0.f;
    }
    if (p.out == nullptr) return;  // forward only: the exp values are not kept
    __syncthreads();
    char* wl = smem + wave * 16384;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int t = 16 * j + c;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const bf16x4 v = {(__bf16)acc[i][j][0], (__bf16)acc[i][j][1], (__bf16)acc[i][j][2], (__bf16)acc[i][j][3]};
        const int chunk = 2 * (i & 3) + (g >> 1);  // ids 16 (i % 4) + 4 g .. + 3 of the tile row
        *(bf16x4*)(wl + (i >> 2) * 8192 + t * 128 + ((chunk ^ (t & 7)) << 4) + 8 * (g & 1)) = v;
      }
    }
    __syncthreads();
    if (nw < p.valid_n) {
      T* tile0 = (T*)p.out + (nw >> 6) * p.ldo + (mw >> 6) * 4096;
#pragma unroll
      for (int sidx = 0; sidx < 16; ++sidx) {
        const int idx = sidx * 64 + lane;
        const int vb = idx >> 9, t = (idx >> 3) & 63, cc = idx & 7;
        if (mw + 64 * vb < p.valid_m) {
          const u32x4 v = *(const u32x4*)(wl + vb * 8192 + t * 128 + ((cc ^ (t & 7)) << 4));
          *(u32x4*)(tile0 + vb * 4096 + t * 64 + cc * 8) = v;
        }
      }
    }
  } else if constexpr (EPI == EPI_LOGITS) {
    // D rows are vocabulary ids (m), columns are tokens (n).  Per token this
    // lane holds 64 of the 128 logits of its wave's slice; its partner lane
    // (lane ^ 32) holds the other 64.  The slice max mx, the exp values
    // P = exp(z - mx) (stored in the tiled layout, element type T) and their
    // fp32 sum are what the row pass needs; the logits themselves are not kept.
    const int slice = (int)(mw / 128);
    T* pout = (T*)p.out;
    // Ids past valid_m take no part in the max and the sum: selects on a
    // 32-bit id for a tile that crosses valid_m, nothing for a full one (a
    // branch per value would cost more than the exponentials).
    const bool mfull = mw + WTM <= p.valid_m;
    const int m0lane = (int)mw + h * 4;
    const int vm = (int)(p.valid_m < (int64_t)0x7FFFFFFF ? p.valid_m : (int64_t)0x7FFFFFFF);
    u32x4 idw[FN];
    uint32_t idpre[FN];
    float gw = 0.f;
    int glive = 0x7FFFFFFF;
    if (p.g_lse != nullptr) grad_weight(p, gw, glive);
    if (p.id_bits != nullptr) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int t = (int)(nw - n0) + 32 * j + col;
        idw[j] = *(const u32x4*)(smem + XOFF + t * 32 + wm * 16);
        idpre[j] = *(const uint32_t*)(smem + XOFF + kIdBitsBytes + 4 * t);
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = nw + j * 32 + col;
      if (p.id_bits != nullptr) {
        // logits at the cached ids of token n in this wave's slice: lane half
        // h holds bits 4 h .. 4 h + 3 of every 8 (block i = bit / 32, slot
        // 4 (bit % 32 / 8) + bit % 4)
        static_assert(FM == 4, "one 32-bit mask word per 32-row block");
        const u32x4 w = idw[j];
        const uint32_t lm = 0x0F0F0F0Fu << (4 * h);
        if (((w.x | w.y | w.z | w.w) & lm) != 0u) {
          uint32_t run = (idpre[j] >> (16 * wm)) & 0xFFFFu;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t word = w[q];
            uint32_t m = word & lm;
            while (m != 0u) {
              const int b = __builtin_ctz(m);
              m &= m - 1u;
              const uint32_t rk = run + (uint32_t)__builtin_popcount(word & ((1u << b) - 1u));
              const float v = pick16(acc[q][j], ((b >> 3) << 2) | (b & 3));
              if (rk < (uint32_t)p.zk) p.zs[n * p.zk + rk] = v;
            }
            run += (uint32_t)__builtin_popcount(word);
          }
        }
      }
      float mx = -INFINITY, sum = 0.f;
      if (mfull) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[i][j][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float nmx = -mx * kLog2e;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = slice_exp<T>(acc[i][j][r], mx, nmx);
            acc[i][j][r] = e;
            sum += e;
          }
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool ok = m0lane + i * 32 + (r >> 2) * 8 + (r & 3) < vm;
            mx = fmaxf(mx, ok ? acc[i][j][r] : -INFINITY);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float nmx = -mx * kLog2e;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool ok = m0lane + i * 32 + (r >> 2) * 8 + (r & 3) < vm;
            const float e = slice_exp<T>(acc[i][j][r], mx, nmx);
            acc[i][j][r] = e;
            sum += ok ? e : 0.f;
          }
      }
      sum += __shfl_xor(sum, 32);
      const bool nvalid = n < p.valid_n;
      if (h == 0 && nvalid && slice < p.n_slices) p.part[n * p.n_slices + slice] = make_float2(mx, sum);
      if (p.g_lse != nullptr) {
        // the gradient's dense part instead of the exp values (zero past V
        // and past the rows)
        const float f = grad_factor(p, n, mx, gw, glive);
        const bool rok = grad_row(p, n, glive);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool ok = m0lane + i * 32 + (r >> 2) * 8 + (r & 3) < vm;
            acc[i][j][r] = (rok && (mfull || ok)) ? f * (float)(T)acc[i][j][r] : 0.f;
          }
      }
      if constexpr (sizeof(T) == 2) continue;  // bf16: stored through LDS below
      if (nvalid && p.out != nullptr) {
        // tile row of token n; the 4 values of (i, q) are consecutive ids
        T* prow = pout + (n >> 6) * p.ldo + (n & 63) * 64;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t m = mw + i * 32 + q * 8 + h * 4;
            if (full || m < p.valid_m) {
              T* dst = prow + (m >> 6) * 4096 + (m & 63);
              if constexpr (sizeof(T) == 2) {
                typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
                bf16x4 v = {(__bf16)acc[i][j][4 * q], (__bf16)acc[i][j][4 * q + 1], (__bf16)acc[i][j][4 * q + 2],
                            (__bf16)acc[i][j][4 * q + 3]};
                *(bf16x4*)dst = v;
              } else {
                f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                *(f32x4*)dst = v;
              }
            }
          }
      }
    }
    if constexpr (sizeof(T) == 2) {
      // The wave's exp values are two whole 64 x 64 tiles of P (tokens nw ..
      // nw + 63, vocabulary mw .. mw + 127), 8 KiB each and contiguous in
      // memory, but a lane holds 4 consecutive ids of one token: stored
      // directly, every wave store would touch 64 lines.  They go through this
      // wave's 16 KiB of LDS (free once every wave has left the main loop) in
      // the tiles' own order, 16-byte chunks of a token row XOR-swizzled by
      // the row, and leave as 16 fully coalesced 1 KiB stores.
      static_assert(WTM == 128 && WTN == 64 && NW * 16384 <= NS * STAGE, "one wave = two 64 x 64 tiles");
      if (p.out == nullptr) return;  // forward only: the exp values are not kept
      __syncthreads();
      char* wl = smem + wave * 16384;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int t = 32 * j + col;  // token row within the tiles
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
            const bf16x4 v = {(__bf16)acc[i][j][4 * q], (__bf16)acc[i][j][4 * q + 1], (__bf16)acc[i][j][4 * q + 2],
                              (__bf16)acc[i][j][4 * q + 3]};
            const int chunk = 4 * (i & 1) + q;  // 16-byte chunk of the token row within tile i / 2
            *(bf16x4*)(wl + (i >> 1) * 8192 + t * 128 + ((chunk ^ (t & 7)) << 4) + 8 * h) = v;
          }
      }
      __syncthreads();
      if (nw < p.valid_n) {
        T* tile0 = pout + (nw >> 6) * p.ldo + (mw >> 6) * 4096;
#pragma unroll
        for (int sidx = 0; sidx < 16; ++sidx) {
          const int idx = sidx * 64 + lane;
          const int vb = idx >> 9, t = (idx >> 3) & 63, cc = idx & 7;
          if (mw + 64 * vb < p.valid_m) {
            const u32x4 v = *(const u32x4*)(wl + vb * 8192 + t * 128 + ((cc ^ (t & 7)) << 4));
            *(u32x4*)(tile0 + vb * 4096 + t * 64 + cc * 8) = v;
          }
        }
      }
    }
  } else {
    float* out = (float*)p.out + (EPI == EPI_SLAB ? (int64_t)tc.split * p.split_stride : 0);
    const bool accum = EPI == EPI_ACCUM && p.beta;
    const int64_t ldo = p.ldo;
    if (full) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        float* rowbase = out + (mw + i * 32 + h * 4) * ldo + nw + col;
        if (accum) {
          // all loads of this row band first, then the adds and stores
          float old[FN][16];
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) old[j][r] = rowbase[((r >> 2) * 8 + (r & 3)) * ldo + j * 32];
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) rowbase[((r >> 2) * 8 + (r & 3)) * ldo + j * 32] = old[j][r] + acc[i][j][r];
        } else {
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) rowbase[((r >> 2) * 8 + (r & 3)) * ldo + j * 32] = acc[i][j][r];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t n = nw + j * 32 + col;
          if (n >= p.valid_n) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t m = mw + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
            if (m < p.valid_m) {
              float* dst = out + m * ldo + n;
              *dst = accum ? *dst + acc[i][j][r] : acc[i][j][r];
            }
          }
        }
    }
  }
}

// ---------------------------------------------------------------- host side
inline int cdiv64(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// One launch over every tile of p; the grid is rounded up to a multiple of
// the 8 XCDs so that each XCD gets the same share of the tile order.
template <typename T, int BM, int BN, int WM, int WN, bool AK, bool BKM, int EPI, int KB, int NS, int MS = 32>
hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  const int total = p.tiles_m * p.tiles_n * p.splits;
  const int grid = ((total + 7) / 8) * 8;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, AK, BKM, EPI, KB, NS, MS>), dim3(grid), dim3(WM * WN * 64), 0,
                     s, p);
  return hipGetLastError();
}

}  // namespace ckl
