// Host side of the pipelined outer-step launch with the lean recurrence
// (casgd_step.h): which (rows, columns) variant a shape runs, the launch's
// LDS and grid, and the dispatch to the variants' translation units.
#include "casgd_train.h"

namespace casgd {

hipError_t launch_step_1x1(int storage, int loss, const PipeArgs& p, int grid, size_t lds, hipStream_t st,
                           const LaunchTimer& tm);
hipError_t launch_step_2x1(int storage, int loss, const PipeArgs& p, int grid, size_t lds, hipStream_t st,
                           const LaunchTimer& tm);
hipError_t launch_step_2x2(int storage, int loss, const PipeArgs& p, int grid, size_t lds, hipStream_t st,
                           const LaunchTimer& tm);
hipError_t launch_step_4x2(int storage, int loss, const PipeArgs& p, int grid, size_t lds, hipStream_t st,
                           const LaunchTimer& tm);
hipError_t launch_step_4x4(int storage, int loss, const PipeArgs& p, int grid, size_t lds, hipStream_t st,
                           const LaunchTimer& tm);

hipError_t launch_train_1x1(int storage, const persist::TrainArgs& A, int grid, size_t lds, hipStream_t st,
                            const LaunchTimer& tm);
hipError_t launch_train_2x1(int storage, const persist::TrainArgs& A, int grid, size_t lds, hipStream_t st,
                            const LaunchTimer& tm);
hipError_t launch_train_2x2(int storage, const persist::TrainArgs& A, int grid, size_t lds, hipStream_t st,
                            const LaunchTimer& tm);
hipError_t launch_train_4x2(int storage, const persist::TrainArgs& A, int grid, size_t lds, hipStream_t st,
                            const LaunchTimer& tm);
hipError_t launch_train_4x4(int storage, const persist::TrainArgs& A, int grid, size_t lds, hipStream_t st,
                            const LaunchTimer& tm);

namespace {

// The smallest variant with at least ceil(b / Q) own rows per minibatch and
// ceil(b / 64) columns per lane.
bool pick(int b, int Q, int& NO, int& CP) {
  static const int kV[5][2] = {{1, 1}, {2, 1}, {2, 2}, {4, 2}, {4, 4}};
  const int nown = (b + Q - 1) / Q, cpl = (b + 63) / 64;
  for (const auto& v : kV)
    if (nown <= v[0] && cpl <= v[1]) {
      NO = v[0];
      CP = v[1];
      return true;
    }
  return false;
}

}  // namespace

bool step_fits(int s, int b, int Q, int64_t ld) {
  (void)ld;
  if (b % 4 != 0 || Q < 1) return false;  // rows of G are copied as float4
  int NO = 0, CP = 0;
  if (!pick(b, Q, NO, CP)) return false;
  return step::layout(s, b, NO, CP).total * static_cast<int64_t>(sizeof(float)) <= step::kLdsBudget;
}

hipError_t launch_step(int storage, int loss, const PipeArgs& p, hipStream_t st, const LaunchTimer& tm) {
  int NO = 0, CP = 0;
  if (!pick(p.a.b, p.a.Q, NO, CP) || p.mar_wgs <= 0 || !p.a.vbox) return hipErrorInvalidValue;
  size_t lds = static_cast<size_t>(step::layout(p.a.s, p.a.b, NO, CP).total) * sizeof(float);
  // the margin workgroups stage w in LDS, the Gram's tiles their stages
  const size_t wl = p.a.ld <= chain::kWlMax ? sizeof(float) * p.a.ld : 0;
  const size_t glds = storage == kStoreF32 ? sizeof(float) * gram::kF32LdsElems
                      : sizeof(uint16_t) * (gram_variant(p.a.ld) == 0 ? gram::lds_elems<32>() : gram::lds_elems<64>());
  if (wl > lds) lds = wl;
  if (p.gram_slots > 0 && glds > lds) lds = glds;
  int others = p.mar0 + p.mar_wgs;
  if (p.gram_slots > 0) others = p.gram0 + p.gram_slots;
  if (p.gath_wgs > 0) others = p.gath0 + p.gath_wgs;
  int grid;
  if (p.a.stride == 1) {
    grid = p.ochain + others;
  } else {
    const int per = p.a.stride - 1;
    const int slots_o = (others + per - 1) / per;
    grid = (slots_o > p.a.Q ? slots_o : p.a.Q) * p.a.stride;
  }
  if (NO == 1) return launch_step_1x1(storage, loss, p, grid, lds, st, tm);
  if (NO == 2 && CP == 1) return launch_step_2x1(storage, loss, p, grid, lds, st, tm);
  if (NO == 2) return launch_step_2x2(storage, loss, p, grid, lds, st, tm);
  if (CP == 2) return launch_step_4x2(storage, loss, p, grid, lds, st, tm);
  return launch_step_4x4(storage, loss, p, grid, lds, st, tm);
}

// LDS of the persistent launch: the chain's layout (with a second G buffer
// when dbl), the margin workgroups' copy of w and their mar_rows rows, the
// Gram's stages.  0 if it does not fit.
size_t train_lds(int storage, int s, int b, int Q, int64_t ld, int mar_rows, bool dbl) {
  int NO = 0, CP = 0;
  if (!pick(b, Q, NO, CP)) return 0;
  const step::Layout L = step::layout(s, b, NO, CP);
  // the chain: its layout, a second G buffer and the update's scratch past
  // both (dbl), then the row indices of two steps
  const int64_t floats = persist::idx_offset(L, NO, dbl, static_cast<int64_t>(s) * NO * L.LW) +
                         2 * ((static_cast<int64_t>(s) * b + 3) & ~3LL) + static_cast<int64_t>(s) * NO;
  size_t lds = static_cast<size_t>(floats) * sizeof(float);
  const size_t esize = storage == kStoreBF16 ? 2 : 4;
  const size_t mlds = sizeof(float) * static_cast<size_t>((ld + 3) & ~3LL) + esize * static_cast<size_t>(ld) * mar_rows;
  const size_t glds = storage != kStoreBF16 ? sizeof(float) * gram::kF32LdsElems
                      : sizeof(uint16_t) * (gram_variant(ld) == 0 ? gram::lds_elems<32>() : gram::lds_elems<64>());
  if (mlds > lds) lds = mlds;
  if (glds > lds) lds = glds;
  return lds <= static_cast<size_t>(step::kLdsBudget) ? lds : 0;
}

hipError_t launch_train(int storage, const persist::TrainArgs& A, int grid, hipStream_t st, const LaunchTimer& tm) {
  int NO = 0, CP = 0;
  if (!pick(A.b, A.Q, NO, CP)) return hipErrorInvalidValue;
  const size_t lds = train_lds(storage, A.s, A.b, A.Q, A.ld, A.mar_rows, A.dbl != 0);
  if (lds == 0) return hipErrorInvalidValue;
  if (NO == 1) return launch_train_1x1(storage, A, grid, lds, st, tm);
  if (NO == 2 && CP == 1) return launch_train_2x1(storage, A, grid, lds, st, tm);
  if (NO == 2) return launch_train_2x2(storage, A, grid, lds, st, tm);
  if (CP == 2) return launch_train_4x2(storage, A, grid, lds, st, tm);
  return launch_train_4x4(storage, A, grid, lds, st, tm);
}

}  // namespace casgd
