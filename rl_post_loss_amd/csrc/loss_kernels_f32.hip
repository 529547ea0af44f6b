// The policy-loss kernels for float log-probs (one translation unit per
// dtype, so that the three tables compile in parallel).
#include "loss_kernels_impl.h"

namespace rlpl {
template const void* pick_typed<float>(int mode, bool has_kl, bool write_grad, int shape);
}  // namespace rlpl
