// Host-side launchers of the device kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckl {

enum Dtype : int { DT_BF16 = 0, DT_F32 = 1 };

// Logits of one chunk: Z[n][v] = H_c[n] . W[v] for n < rows, v < V (fp32, row
// stride ldz), and per (row, 128-vocabulary slice) the pair (max, sum exp).
hipError_t launch_logits(Dtype dt, const void* W, const void* Hc, int64_t V, int64_t d, int64_t rows,
                         float* Z, int64_t ldz, float2* part, int n_slices, hipStream_t s);

// dH partial slabs of one chunk: slab[s][n][j] = sum over the s-th vocabulary
// split of G[n][v] W[v][j].  G has row stride ldg elements of the type.
hipError_t launch_dh(Dtype dt, const void* G, int64_t ldg, const void* W, int64_t V, int64_t d, int64_t rows,
                     float* slab, int splits, hipStream_t s);
// dH rows = sum of the slabs in split order, rounded once to the output type.
hipError_t launch_dh_reduce(Dtype dt, const float* slab, int splits, int64_t rows, int64_t d, void* dH,
                            hipStream_t s);
// dW (+)= G^T H_c over the rows of one chunk; beta = 0 overwrites.
hipError_t launch_dw(Dtype dt, const void* G, int64_t ldg, const void* Hc, int64_t V, int64_t d, int64_t rows,
                     float* dW, int beta, hipStream_t s);

// k-splits used for the dH contraction of a chunk of `rows` rows.
int dh_splits(int64_t rows, int64_t d, int64_t V);
// tile width used along d by the dH and dW contractions.
int d_tile(int64_t d);

// Valid-token count n and scale 1/n (0 if n = 0) into scal (int64 n, float s).
hipError_t launch_mask_count(const uint8_t* mask, int64_t N, void* scal, hipStream_t s);

// Row pass of one chunk: lse from the partials, teacher softmax, gather, KL,
// in-place gradient G = w (softmax - scatter(p_T)) over the Z rows.
struct RowArgs {
  float* Z;
  int64_t ldz;          // fp32 elements per Z row
  const float2* part;   // per row n_slices pairs (max, sum exp)
  int n_slices;
  const int32_t* ids;   // [rows, K]
  const float* tlogit;  // [rows, K]
  const uint8_t* mask;  // [rows] or null
  const void* scal;     // device scalars (int64 n, float s); null -> scale_value
  float scale_value;
  int64_t V;
  int K;
  int64_t rows;
  float* kl_out;        // [rows] KL (0 for masked rows)
  float* lse_out;       // [rows]
  float* zg_dbg;        // optional [rows, K]
  int32_t* sid_dbg;     // optional [rows, K]
};
hipError_t launch_rows(Dtype g_dt, const RowArgs& a, hipStream_t s);

// Debug helper: partials of caller-given Z rows (same slicing as the logits kernel).
hipError_t launch_partials_from_z(const float* Z, int64_t ldz, int64_t rows, int64_t V, float2* part,
                                  int n_slices, hipStream_t s);

// loss = s * sum of kl[0..N) in a fixed order, accumulated in double.
hipError_t launch_finalize(const float* kl, int64_t N, const void* scal, float* out_loss, hipStream_t s);

constexpr int kMaxK = 2048;

}  // namespace ckl
