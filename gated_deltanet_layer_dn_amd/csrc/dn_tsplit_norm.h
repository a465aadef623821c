// The out_proj input split of the prefill path with the gated RMSNorm applied first (page "qwen36:
// run the DeltaNet layer end to end on the card", section "What the PR does", Backend paragraph:
// the gated RMSNorm with silu(z), per value head over the readout).
// Per head of 128 columns: y = w o / sqrt(mean o^2 + eps) silu(z), then the three-term int8 split
// of each token's row y, as launch_tsplit does for an unnormalised row.
#pragma once
#include "dn_internal.h"

namespace dn {

struct TSplitNormArgs {
  TSplitArgs sp;        // act = the readout o [T][act_stride]; K = heads x 128, at most 8192
  const float* z;       // [T][z_stride], the gate's pre-activations, 16-byte aligned
  int z_stride;
  const float* norm_w;  // [128]
  float eps;
};
hipError_t launch_tsplit_norm(const TSplitNormArgs& a, hipStream_t st);

}  // namespace dn
