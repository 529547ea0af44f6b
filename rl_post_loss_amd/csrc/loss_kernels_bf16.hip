// The policy-loss kernels for __bf16 log-probs (one translation unit per
// dtype, so that the three tables compile in parallel).
#include "loss_kernels_impl.h"

namespace rlpl {
template const void* pick_typed<__bf16>(int mode, bool has_kl, bool write_grad, int shape);
}  // namespace rlpl
