// Decode-path picker: an estimate of one decode step of each GQLA path on MI355X, from
// the work this library's kernels do and throughputs measured for them on that GPU.
//
// The pages' point is that the two algebraically equal forms trade cache traffic for
// computation and that which one wins depends on the hardware ("GQLA: Attention latente
// ...", English abstract; the decode_path switch of gqla_attn.py; the H20-3e comparison in
// "GQLA: Group-Query Latent Attention for Hardware-Adaptive Decoding", Abstract, and in
// "GQLA: Новая архитектура внимания адаптирует LLM под разное железо без переобучения"):
// the MQA-absorb path reads d_c + d_R values per token but does H * s_q dense
// head-products over them; the GQA path reads G * (d_qk + d_v) values per token with only
// 16-row MFMA tiles per group. MI355X has H100-like balance (8 TB/s, 2.5 PFLOP/s bf16),
// so the crossover sits far from the H20's.
#include "../../include/gqla.h"
#include "gqla_internal.h"
#include "tuned.h"

#include <algorithm>
#include <cmath>

namespace gqla {

// Effective throughputs of the kernels in this library, MI355X, bf16 (measured with
// bench.py and the crossover sweep; see the path-crossover profile).
// Each decode also has a fixed cost that does not shrink with the context: the first tile's
// fetch before any compute, the partial-output stores, and the last workgroups' tail
// (~15 us for the absorb decode by per-workgroup timestamps on LLaMA-3-8B batch 32).
struct Mi355xRates {
  double absorb_bw = 6.2e12;      // absorb decode latent streaming, B/s (tile copies into LDS)
  double absorb_mfma = 0.9e15;    // absorb decode when MFMA/LDS-bound, flop/s (specialized waves)
  double absorb_fixed_us = 15.0;  // absorb decode fixed cost
  double gqa_bw = 6.8e12;         // GQA decode expanded-cache streaming, B/s (per-group layout)
  double gqa_shared_bw = 7.0e12;  // same, RoPE key once per block
  double gqa_fixed_us = 20.0;     // GQA step fixed cost (decode and new-token expansion)
  double gqa_mfma = 1.0e15;       // GQA decode padded MFMA work, flop/s
  double expand_mfma = 0.35e15;   // cache expansion, flop/s
  double proj_mfma = 0.2e15;      // absorbed-query and value projections, flop/s
  double combine_bw = 3.0e12;     // split combine, B/s of partial results
  double launch_us = 3.0;         // fixed cost per kernel in a back-to-back step
};

PathEstimate estimate_paths(const gqla_dims* d, int64_t total_ctx, int n_split_abs, int n_split_gqa) {
  const Mi355xRates r;
  const double B = d->batch, H = d->num_heads, G = d->num_groups, s = d->s_q;
  const double dc = d->latent_rank, dr = d->rope_dim, dn = d->nope_dim, dv = d->v_dim;
  const double dqk = dn + dr;
  const double elt = d->dtype == GQLA_BF16 ? 2.0 : 4.0;
  const double tok = static_cast<double>(total_ctx);
  // Query-token pairs: row i of sequence b sees L_b - s_q + 1 + i tokens.
  const double vis = s * tok - B * s * (s - 1.0) / 2.0;
  const double rows = B * s * H;
  auto us = [](double x) { return x * 1e6; };

  // MQA-absorb: absorbed query, latent decode, value projection (split: one kernel that
  // merges the partials and applies W_UV^g, as gqla_decode_absorb_out runs it).
  const double abs_bytes = tok * (dc + dr) * elt;
  const double abs_flops = vis * H * 2.0 * (2.0 * dc + dr);
  double t_abs = std::max(us(abs_bytes / r.absorb_bw), us(abs_flops / r.absorb_mfma)) + r.absorb_fixed_us;
  t_abs += 2 * r.launch_us + us(rows * dn * dc * 2.0 / r.proj_mfma) + us(rows * dc * dv * 4.0 / r.proj_mfma);
  if (n_split_abs > 1) t_abs += us(rows * n_split_abs * dc * 4.0 / r.combine_bw);

  // GQA: expansion of the blocks holding the new tokens, grouped decode, (combine).
  const double gqa_bytes = tok * (d->rope_shared ? G * (dn + dv) + dr : G * (dqk + dv)) * elt;
  const double tile_rows = 16.0 * std::ceil(H / G * s / 16.0);
  const double gqa_flops = tok * G * tile_rows * 2.0 * (dqk + dv);
  const double gqa_bw = d->rope_shared ? r.gqa_shared_bw : r.gqa_bw;
  double t_gqa = std::max(us(gqa_bytes / gqa_bw), us(gqa_flops / r.gqa_mfma)) + r.gqa_fixed_us;
  const double new_blocks = B * (1.0 + (s - 1.0) / kBlock);
  t_gqa += r.launch_us + us(new_blocks * G * kBlock * (dn + dv) * dc * 2.0 / r.expand_mfma);
  if (n_split_gqa > 1) t_gqa += r.launch_us + us(B * s * H * n_split_gqa * dv * 4.0 / r.combine_bw);
  return {t_abs, t_gqa};
}

}  // namespace gqla
