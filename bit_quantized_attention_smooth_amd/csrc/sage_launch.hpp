// sage_launch.hpp -- host-side launchers of the HIP kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sage {

enum { QK_INT8 = 1, QK_MXFP4 = 3 };
enum { PV_FP8 = 2, PV_MXFP4 = 3, PV_MXFP8 = 4 };

// Padding of the token axis in every quantized buffer (a multiple of the Q tile).
constexpr int kTokenPad = 128;
// Token chunks per head of the smoothing statistics (partial sums are kept per chunk).
constexpr int kStatChunks = 8;

// Device pointers of one quantized buffer (offsets resolved on the host).
struct QuantPtrs {
  float* mu_k;
  float* mu_q;
  uint8_t* q_codes;
  void* q_scales;     // fp32 [BH, nb] (INT8) or uint8 E8M0 [BH, Np, d/32] (MXFP4)
  uint8_t* k_codes;
  void* k_scales;
  uint8_t* v_codes;
  void* v_scales;     // fp32 [BH, d] (FP8) or uint8 E8M0 [BH, Np/32, d] (MXFP4, MXFP8)
  float* delta_s;
  float* lse_corr;
  double* sums;       // [2, BH, d]: K then Q token sums
  uint32_t* amax_v;   // [BH, d] bit patterns of max |V| per channel
};

struct Shape {
  int B, H, N, d, Np, causal, io_dtype, qk_fmt, pv_fmt;
  float sm_scale;
};

hipError_t launch_prologue(const void* q, const void* k, const void* v, const Shape& s,
                           const QuantPtrs& qp, hipStream_t stream);
hipError_t launch_attn_fwd(const Shape& s, const QuantPtrs& qp, void* o, float* lse, hipStream_t stream);

// Backward: the workspace is [forward quant buffer (qbytes) | backward extras];
// attn_bwd_ws_bytes gives the size of the extras.  Head dim 64 only.
size_t attn_bwd_ws_bytes(const Shape& s);
hipError_t launch_attn_bwd(const Shape& s, const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, void* ws,
                           size_t qbytes, const QuantPtrs& qp, hipStream_t stream);

}  // namespace sage
