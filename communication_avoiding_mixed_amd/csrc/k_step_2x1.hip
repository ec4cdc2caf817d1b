// The 2-row, 1-column-per-lane variant of the pipelined outer-step
// launch (casgd_step.h), in a translation unit of its own so the variants
// compile in parallel.
#include "casgd_train.h"

namespace casgd {

hipError_t launch_step_2x1(int storage, int loss, const PipeArgs& p, int grid, size_t lds, hipStream_t st,
                           const LaunchTimer& tm) {
  return step::launch_variant<2, 1>(storage, loss, p, grid, lds, st, tm);
}

hipError_t launch_train_2x1(int storage, const persist::TrainArgs& A, int grid, size_t lds, hipStream_t st,
                            const LaunchTimer& tm) {
  return persist::launch_variant<2, 1>(storage, A, grid, lds, st, tm);
}

}  // namespace casgd
