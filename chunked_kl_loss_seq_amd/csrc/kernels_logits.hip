// Launcher of the logits contraction with its fused exp epilogue.  Both of its
// operands are contiguous along d, so the bf16 path runs on 16 x 16 x 32 MFMA
// blocks, which sustain a higher rate than 32 x 32 x 16 under the board's power
// limit; the fp32 path keeps 32 x 32 blocks.
#include "gemm_core.hpp"
#include "launch.hpp"

namespace ckl {

hipError_t launch_logits(Dtype dt, const void* Wt, const void* Hc, int64_t V, int64_t d, int64_t rows, void* P,
                         int64_t pblk, float2* part, int n_slices, const IdTables* tab, const GradTerms* grad,
                         const int* live, hipStream_t s) {
  GemmParams p{};
  p.live = live;
  p.a = Operand{Wt, 0, V, d, tile_row_stride(d)};  // tiled: storage row = vocabulary id, column = d
  p.b = Operand{Hc, d, rows, d, 0};
  p.tiles_m = cdiv64(V, 256);
  p.tiles_n = cdiv64(rows, 256);
  const int bk = dt == DT_BF16 ? 64 : 32;
  p.k_tiles = cdiv64(d, bk);
  p.splits = 1;
  p.k_tiles_per_split = p.k_tiles;
  p.group_m = 4;
  p.out = P;
  p.ldo = pblk;
  p.valid_m = V;
  p.valid_n = rows;
  p.part = part;
  p.n_slices = n_slices;
  if (grad != nullptr) {
    p.g_lse = grad->lse;
    p.g_rowmap = grad->rowmap;
    p.g_scale = grad->scale;
    p.g_gscale = grad->gscale;
  }
  if (tab != nullptr) {
    p.id_bits = tab->bits;
    p.id_pre = tab->pre;
    p.id_cpad = tab->cpad;
    p.zs = tab->zs;
    p.zk = tab->K;
  }
  if (dt == DT_BF16) return launch_gemm<__bf16, 256, 256, 2, 4, true, true, EPI_LOGITS, 128, 2, 16>(p, s);
  return launch_gemm<float, 256, 256, 2, 4, true, true, EPI_LOGITS, 128, 2>(p, s);
}

}  // namespace ckl
