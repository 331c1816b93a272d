// cos/sin table builder ("RoPE, scaling, sliding window, attention sinks",
// _compute_cos_sin_cache and its YaRN variant): cell (m, i) holds
// mu cos(m w_i) and mu sin(m w_i), the angle and the trig in fp64, one
// rounding to fp32.  Every cell is computed on its own, so the table is
// bitwise the same for any grid ("--rope-scaling dynamic": the table).
#include "kernels.hpp"

namespace ropekv {

__global__ __launch_bounds__(256) void table_kernel(RopeParams rp, int max_pos, float *__restrict__ out,
                                                    float *mscale_dev) {
  __shared__ double w[256];
  const int half = rp.rotary_dim / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x) w[i] = rope_omega(rp, i);
  __syncthreads();
  const double mu = params_mscale(rp);
  const long total = (long)max_pos * half;
  for (long c = (long)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += (long)gridDim.x * blockDim.x) {
    const long m = c / half;
    const int i = (int)(c - m * half);
    const double ang = (double)m * w[i];
    double sn, cs;
    sincos(ang, &sn, &cs);
    out[m * rp.rotary_dim + i] = (float)(cs * mu);
    out[m * rp.rotary_dim + half + i] = (float)(sn * mu);
  }
  if (mscale_dev && blockIdx.x == 0 && threadIdx.x == 0) *mscale_dev = (float)mu;
}

hipError_t launch_build_table(const RopeParams &rp, int max_pos, float *out, float *mscale_dev, hipStream_t s) {
  const long total = (long)max_pos * (rp.rotary_dim / 2);
  long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(table_kernel, dim3((unsigned)blocks), dim3(256), 0, s, rp, max_pos, out, mscale_dev);
  return hipGetLastError();
}

}  // namespace ropekv
