// Internal interface between the C ABI (lce_api.cpp) and the kernel launchers
// (lce_kernels.hip). Not installed; not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

constexpr int kMaxShards = 256;

// Device pointers of all vocabulary shards, passed by value as a kernel
// argument (2 KB) so no host->device copy is needed.
struct ShardTable {
  const uint16_t* p[kMaxShards];
};

hipError_t launch_fwd_round(const uint16_t* X, int N, int H, const uint16_t* W, int Vs, float2* state, int state_ld,
                            int token_blocks, int S, int tiles_per_split, int n_vtiles, int first, hipStream_t st);
hipError_t launch_target_logit(const uint16_t* X, int N, int H, const ShardTable& shards, int Vs, int V,
                               const int* targets, int ignore_index, float* yt, hipStream_t st);
hipError_t launch_finalize(const float2* state, int state_ld, int S, const float* yt, const int* targets, int N,
                           int ignore_index, float* lse, float* token_loss, double2* partials, int reduction,
                           float* loss, float* n_valid_out, hipStream_t st);
hipError_t launch_bwd_scale(const int* targets, int N, int ignore_index, const float* dloss, int reduction,
                            float* gscale, hipStream_t st);
hipError_t launch_bwd_g(const uint16_t* X, int N, int H, const uint16_t* Ws, int Vs, int v0, int vc, int n0, int nc,
                        const int* targets, const float* lse, const float* gscale, int ignore_index, int vocab_base,
                        int V, uint16_t* G, int ldg, int nc_pad, int vc_pad, hipStream_t st);
hipError_t launch_grad_gemm(const uint16_t* G, int ldg, int nc_pad, int vc_pad, const uint16_t* Wc, int vc,
                            const uint16_t* Xc, int nc, int H, float* dX, int acc_dx, float* dW, int acc_dw,
                            hipStream_t st);

}  // namespace lce
