// attn_launch.h -- internal interface between the C ABI (attn_abi.hip) and the
// gfx950 kernels (attn_kernels.hip).  Arguments arrive here validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nss {

struct FwdArgs {
  const void *q, *k, *v;
  void* o;
  float* o32;  // optional: O before its bf16 rounding, fp32 [B][H][N][D]
  float* lse;
  int32_t *ties, *pbar_one, *formed_ones;
  float* rowmax;
  int B, H, N, D;
  float scale;
  int causal, stabilise;  // stabilise: 0 plain, 1 online duplicate-max shift, 2 exact final shift
  float beta;
};

struct BwdArgs {
  const void *q, *k, *v, *o, *dO;
  const float* o32;  // optional: delta from this fp32 O instead of o
  const float* lse;
  void *dq, *dk, *dv;
  float* delta;
  int B, H, N, D;
  float scale;
  int causal;
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st);
hipError_t launch_tiecount(const FwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t st);
// keys per KV tile of the forward for head size D (0 for an unsupported D)
int fwd_key_tile(int D);

}  // namespace nss
