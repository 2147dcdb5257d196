// Launch interface of the temperature-1 verification kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace dflash {

struct SampledArgs {
  const float* draft_logits;   // [B][15][V]
  const float* target_logits;  // [B][16][V]
  const float* u_draft;        // [B][15]
  const float* u_accept;       // [B][15]
  const float* u_resample;     // [B]
  int vocab;
  double* stats;               // [B][31][2] workspace: (max, sum exp) per row, fp64
  int* draft_ids;              // [B][15]
  int* accept_len;             // [B]
  int* emitted;                // [B][16]
};

hipError_t launch_verify_sampled(const SampledArgs& a, int batch, hipStream_t stream);

}  // namespace dflash
