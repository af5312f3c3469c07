// Forward sweep: the launcher, and the variants with a bias or without the
// grad_h accumulator, compiled with the default scheduler and no per-k-step
// fence (with a bias, the ILP strategy and the fence cost 11 %).
#include "fwd_sweep.h"

namespace plp {

hipError_t launch_fwd_mfma(const __bf16* h, const __bf16* Wf, const __bf16* b, int64_t N, int H, int V, float inv_tau,
                           int Sv, bool with_o, RowStats* stats, float* O, hipStream_t st) {
  if (with_o && !b) return launch_fwd_mfma_o_nobias(h, Wf, N, H, V, inv_tau, Sv, stats, O, st);
  if (with_o) return fwd_launch<true, true, false>(h, Wf, b, N, H, V, inv_tau, Sv, stats, O, st);
  if (b) return fwd_launch<false, true, false>(h, Wf, b, N, H, V, inv_tau, Sv, stats, O, st);
  return fwd_launch<false, false, false>(h, Wf, b, N, H, V, inv_tau, Sv, stats, O, st);
}

}  // namespace plp
