// Per-token MXFP8 quantization of bf16 activations (the w4a8 FC1 input) as
// its own launch: the situ_moe_quantize_mxfp8 entry point.  Inside the layer
// the routing launch quantizes beside the router (route.hip); both run
// quant_mxfp8_piece (quant.hpp), so their codes and scales are the same.
#include "quant.hpp"

namespace situ {

__global__ __launch_bounds__(256) void quant_mxfp8_kernel(QuantArgs a) {
  quant_mxfp8_piece(a, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

hipError_t launch_quant_mxfp8(const QuantArgs& a, hipStream_t s) {
  const int64_t n8 = quant_pieces(a);
  if (n8 == 0) return hipSuccess;
  const int64_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL(quant_mxfp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace situ
