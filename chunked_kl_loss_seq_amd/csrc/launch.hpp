// Host-side launchers of the device kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckl {

enum Dtype : int { DT_BF16 = 0, DT_F32 = 1 };

// Elements between two 64-row tile rows of a 64 x 64-tiled matrix with V columns.
inline int64_t tile_row_stride(int64_t V) { return ((V + 63) / 64) * 4096; }

// Copy of a row-major [rows, cols] matrix (cols % 8 == 0) into the 64 x 64
// tiled layout, tile rows tile_row_stride(cols) elements apart.
hipError_t launch_tile_copy(Dtype dt, const void* src, int64_t rows, int64_t cols, void* dst, hipStream_t s);

// With a mask, a chunk is compacted first (launch_compact) and its kernels
// take `live`: a device int, the number of valid rows, which sit at the front
// of the chunk's buffers.  Rows at and after it are skipped: no logits, zero
// gradient rows.  Without a mask `live` is null and every row is computed.

// Tables of a chunk's cached ids, built by launch_id_tables and read by the
// logits contraction, which copies the fp32 logit at every cached id out of
// its accumulators before they become exp values.
// Layout by vocabulary tile: "pair" p = slices 2p, 2p + 1 = ids 256 p .. 256 p + 255.
struct IdTables {
  const void* bits;    // [pairs][cpad][2] 128-bit masks: bit b of (p, n, h) = id 256 p + 128 h + b is cached for row n
  const void* pre;     // [pairs][cpad] two uint16: distinct cached ids of row n below ids 256 p and 256 p + 128
  int64_t cpad;        // rows of the tables: the chunk's rows rounded up to a multiple of 256
  const int32_t* rank; // [rows][K]: rank of cached id k among its row's distinct ids, -1 if outside [0, V)
  float* zs;           // [rows][K]: logit of the cached id of rank q at zs[n][q]
  int K;
};
inline int64_t id_table_pairs(int64_t V) { return (V + 255) / 256; }

// Id tables of `rows` rows of cached ids [rows, K] (cpad >= rows, a multiple
// of 256); with live (compacted chunk), rows at and past *live get empty
// tables.  Ids outside [0, V) set bit 0 of *err, an id repeated within a row
// bit 1 (err may be null); both are left out of the tables, so no kernel
// reads or writes at them.
hipError_t launch_id_tables(const int32_t* ids, int K, int64_t rows, int64_t V, const int* live, void* bits,
                            void* pre, int64_t cpad, int32_t* rank, unsigned* err, hipStream_t s);

// The recomputing backward knows each row's log-normaliser before its logits:
// the logits epilogue then stores the gradient's dense part itself.
struct GradTerms {
  const float* lse;     // [rows] log-normalisers of the chunk's rows
  const int* rowmap;    // compacted chunk: chunk row of each compacted row (lse index), or null
  const float* scale;   // device scalar 1 / n_valid
  const float* gscale;  // device scalar multiplying the gradient, or null
};

// Logits of one chunk, kept as exp values: per (row n < rows, 128-id slice s)
// the slice max m and sum of exp(z - m) into part[n][s], and exp(z - m) for
// every z = H_c[n] . W[v] into P (element type of dt, tiled, tile rows pblk
// elements apart).  With tab, the fp32 logit at every cached id also goes to
// tab->zs.  P may be null (the forward alone): no exp values are stored.
// With grad, P receives w exp(m - lse) exp(z - m) instead, exactly
// as launch_dense would leave it (w = scale (x gscale) for the rows, 0 past
// them and past V).
// W is the tiled copy of the weight (tile_row_stride(d) elements between tile rows).
hipError_t launch_logits(Dtype dt, const void* Wt, const void* Hc, int64_t V, int64_t d, int64_t rows, void* P,
                         int64_t pblk, float2* part, int n_slices, const IdTables* tab, const GradTerms* grad,
                         const int* live, hipStream_t s);

// dH partial slabs of one chunk: slab[s][n][j] = sum over the s-th vocabulary
// split of G[n][v] W[v][j].  G is tiled like P, tile rows gblk elements apart;
// Wt is the tiled copy of the weight.
hipError_t launch_dh(Dtype dt, const void* G, int64_t gblk, const void* Wt, int64_t V, int64_t d, int64_t rows,
                     float* slab, int splits, const int* live, hipStream_t s);
// dH rows = sum of the slabs in split order, rounded once to the output type.
// With pos (compacted chunk), dH row j takes slab row pos[j], or zeros if -1.
hipError_t launch_dh_reduce(Dtype dt, const float* slab, int splits, int64_t rows, int64_t d, const int* pos,
                            void* dH, hipStream_t s);
// dW (+)= G^T H_c over the rows of one chunk; beta = 0 overwrites.
hipError_t launch_dw(Dtype dt, const void* G, int64_t gblk, const void* Hc, int64_t V, int64_t d, int64_t rows,
                     float* dW, int beta, const int* live, hipStream_t s);

// k-splits used for the dH contraction of a chunk of `rows` rows.
int dh_splits(Dtype dt, int64_t rows, int64_t d, int64_t V);
// The largest split count <= s that cuts the dH k-steps into exactly that many
// runs (what launch_dh requires).
int dh_fit_splits(Dtype dt, int64_t V, int s);
// tile width used along d by the dH and dW contractions.
int d_tile(Dtype dt, int64_t d);

// Per row of x [N, V] (bf16 or fp32), the K largest values and their ids, by
// value descending and equal values by id ascending (see kernels_topk.hip).
hipError_t launch_topk(Dtype dt, const void* x, int64_t N, int64_t V, int64_t K, int32_t* ids, float* vals,
                       hipStream_t s);

// Valid-token count n and scale 1/n (0 if n = 0) into scal (int64 n, float s).
hipError_t launch_mask_count(const uint8_t* mask, int64_t N, void* scal, hipStream_t s);
// Compaction of the chunk whose mask, H rows, ids and teacher logits start at
// the given pointers (`rows` positions): vidx[i] = the chunk row of the i-th
// valid one, pos[j] = the compact index of row j or -1, *live = the valid
// count; masked rows' kl_out (and lse_out, if not null) are set to 0; the
// valid rows of H, ids and logits are gathered to Hc, ids_c, tl_c (chunk
// buffers of rows_alloc rows), and Hc rows [*live, next multiple of 256) are
// zeroed.
hipError_t launch_compact(Dtype dt, const uint8_t* mask, int64_t rows, int64_t rows_alloc, const void* H,
                          int64_t d, const int32_t* ids, const float* tlogit, int K, int* vidx, int* pos,
                          int* live, float* kl_out, float* lse_out, void* Hc, int32_t* ids_c, float* tl_c,
                          hipStream_t s);

// Row pass of one chunk (see kernels_rows.hip).
struct RowArgs {
  void* P;              // tiled exp values in, gradient out (element type of the path)
  int64_t pblk;         // elements between tile rows of P
  float2* part;         // per row n_slices pairs: (max, sum exp) in, (max, gradient factor) out
  int n_slices;
  const int32_t* ids;   // [rows, K]
  const float* tlogit;  // [rows, K]
  const uint8_t* mask;  // [rows] or null
  const void* scal;     // device scalars (int64 n, float s); null -> scale_value
  float scale_value;
  int64_t V;
  int K;
  int64_t rows;
  float* scat;          // [rows, K] exact gradient values at the cached ids
  const float* lse_in;  // [rows] log-normalisers saved by a forward pass, or null: merge the slice pairs
  const float* gscale;  // device scalar multiplying the gradient, or null for 1
  const int* live;      // compacted chunk: rows at and after *live are skipped; null: none
  const int* vidx;      // compacted chunk: chunk row of each compacted row (row outputs, lse_in); or null
  float* kl_out;        // [rows] KL (0 for masked rows), or null
  float* lse_out;       // [rows] log-normalisers, or null
  const int32_t* rank;  // [rows, K] rank of each cached id among its row's distinct ids (-1: outside [0, V))
  const float* zs;      // [rows, K] exact logits of the cached ids, by rank
  float* zg_dbg;        // optional [rows, K]
  int32_t* sid_dbg;     // optional [rows, K]
};
hipError_t launch_row_stats(Dtype g_dt, const RowArgs& a, hipStream_t s);
// p[0 .. n) = v (a kernel, not a memset node, so that the call stays capturable)
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);
hipError_t launch_dense(Dtype g_dt, const RowArgs& a, hipStream_t s);
hipError_t launch_scatter(Dtype g_dt, const RowArgs& a, hipStream_t s);

// Debug helpers: slice pairs and tiled exp values of caller-given fp32 logits
// (row stride ldz); and a tiled matrix copied out to row-major [rows, V].
hipError_t launch_partials_from_z(Dtype g_dt, const float* Z, int64_t ldz, int64_t rows, int64_t V, float2* part,
                                  int n_slices, void* P, int64_t pblk, hipStream_t s);
// Debug helper: zs[r][rank[r][k]] = Z[r][ids[r][k]] for the ids of the table.
hipError_t launch_zs_from_z(const float* Z, int64_t ldz, const int32_t* ids, const int32_t* rank, int64_t rows, int K,
                            float* zs, hipStream_t s);
hipError_t launch_untile(Dtype g_dt, const void* P, int64_t pblk, int64_t rows, int64_t V, void* out,
                         hipStream_t s);

// loss = s * sum of kl[0..N) in a fixed order, accumulated in double.
hipError_t launch_finalize(const float* kl, int64_t N, const void* scal, float* out_loss, hipStream_t s);

constexpr int kMaxK = 2048;
// byte offsets, in the device scalar block, of the gradient weight 1 / n_valid
// (fp32) and of the input-check flags (bit 0: a cached id outside [0, V);
// bit 1: an id repeated within a row)
constexpr int kScaleOffset = 8;
constexpr int kErrOffset = 16;

}  // namespace ckl
