// gate_prologue.hip -- the gate prologue on its own:
//     g = -exp(A_log) * softplus(a + dt_bias),   beta = sigmoid(b)
// per (token, value head), in float32, narrowed once to the I/O dtype.
// Pages: [P1] onnxruntime-ep-mlx, src/ops/ssm.rs, `linear_attention_gate_op`
// (softplus of a + bias times a per-head decay scale, sigmoid of b);
// [P4] onnx-runtime-ep-cuda, src/kernels/linear_attention.rs, the fused
// gate branch of `linear_attention_core` and its helpers.
// Elementwise and HBM-bound: grid-stride over rows * h_v elements.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

template <typename IO>
__global__ __launch_bounds__(256) void gate_kernel(GatePrologueParams p) {
  const int64_t total = p.rows * p.h_v;
  const IO* a = static_cast<const IO*>(p.a);
  const IO* b = static_cast<const IO*>(p.b);
  IO* g = static_cast<IO*>(p.g);
  IO* beta = static_cast<IO*>(p.beta);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int h = static_cast<int>(e % p.h_v);
    if (g != nullptr) narrow_store(g + e, gate_log_decay(widen(a[e]), p.A_log[h], p.dt_bias[h]));
    if (beta != nullptr) narrow_store(beta + e, gate_sigmoid(widen(b[e])));
  }
}

}  // namespace

hipError_t launch_gate_prologue(GatePrologueParams p, int io_dtype, hipStream_t stream) {
  const int64_t total = p.rows * p.h_v;
  if (total == 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 4096 ? want : 4096);
  if (io_dtype == 1)
    hipLaunchKernelGGL((gate_kernel<bf16_t>), dim3(blocks), dim3(256), 0, stream, p);
  else if (io_dtype == 2)
    hipLaunchKernelGGL((gate_kernel<f16_t>), dim3(blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((gate_kernel<float>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gdn
