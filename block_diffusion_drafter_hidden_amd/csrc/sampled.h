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
  double* chunk_sums;          // [B][chunks_ld] workspace: sums of the final draw's weights
                               // over each 256-element chunk of its row
  int chunks_ld;               // ceil(V / 256)
  float* picks;                // [B][15][2] workspace: each drawn draft token's draft and
                               // target logits
  int* draft_ids;              // [B][15]
  int* accept_len;             // [B]
  int* emitted;                // [B][16]
  double exp_k[4];             // set by launch_verify_sampled: log2(e) and the fp64
                               // coefficients of 2^f (kernel arguments live in scalar
                               // registers, which the fp64 fma takes directly)
};

// Largest vocabulary of the temperature-1 verify: 4096 chunks of 256 logits, whose
// statistics a workgroup keeps in 48 KB of LDS.
constexpr int kMaxSampledVocab = 4096 * 256;

hipError_t launch_verify_sampled(const SampledArgs& a, int batch, hipStream_t stream);
// Workspace bytes of launch_verify_sampled (row statistics, chunk sums, picked logits).
size_t verify_sampled_stats_bytes(int batch, int vocab);

}  // namespace dflash
