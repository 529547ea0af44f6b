// The policy-loss kernels for _Float16 log-probs (one translation unit per
// dtype, so that the three tables compile in parallel).
#include "loss_kernels_impl.h"

namespace rlpl {
template const void* pick_typed<_Float16>(int mode, bool has_kl, bool write_grad, int shape);
}  // namespace rlpl
