// Per-output-channel FP8 (OCP E4M3) quantisation of expert weights.
//
// The page on MoE latency (wink.run), in its section on what to do about the
// cost, names quantising weights as a way to move fewer bytes and asks that
// the numerical error be measured.  The format and the scale rule are this
// library's reading: OCP E4M3 (bias 7, subnormals m * 2^-9, largest finite
// 448, no infinity) with one float32 scale per output channel,
//   scale[r] = max_k |w[r][k]| / 448    (1 for an all-zero row),
//   q[r][k]  = E4M3 nearest to w[r][k] / scale[r], ties to the even code,
//              magnitudes >= 448 saturated, sign kept.
// Both divisions are taken in double and rounded once to float32, which
// equals the correctly rounded float32 quotient (53 >= 2 * 24 + 2 bits).
// Weights are quantised once, ahead of inference; this is not on the layer's
// path.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr float kE4M3Max = 448.f;

// E4M3 code of a float32, from the format's definition.  Normal range
// [2^-6, 448): the exponent field is the float's minus 120 and the three
// mantissa bits are the float's top three, rounded half to even on the 20
// dropped bits (a carry moves into the exponent, which is the next code).
// Below 2^-6 the values are the multiples of 2^-9: the code is
// rint(a * 512) (8 = the smallest normal, code 0x08).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (!(a < kE4M3Max)) {
    code = 0x7Eu;                                // saturate (also 448 itself)
  } else if (a < 0x1p-6f) {
    code = (uint32_t)rintf(a * 512.f);
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    code = (b >> 20) - (120u << 3);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// One block of 256 threads per row (grid-stride over rows); eight weights per
// thread per step.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* __restrict__ w, long long rows,
                                                           int cols, uint8_t* __restrict__ q,
                                                           float* __restrict__ scale) {
  __shared__ float s_max[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (long long r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint16_t* src = w + r * cols;
    float m = 0.f;
    for (int c = tid * 8; c < cols; c += 256 * 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + c);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m = fmaxf(m, fabsf(__uint_as_float(u[j] << 16)));
        m = fmaxf(m, fabsf(__uint_as_float(u[j] & 0xFFFF0000u)));
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
    if (lane == 0) s_max[wave] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const float sc = amax > 0.f ? (float)((double)amax / (double)kE4M3Max) : 1.f;
    if (tid == 0) scale[r] = sc;
    const double dsc = (double)sc;
    uint8_t* dst = q + r * cols;
    for (int c = tid * 8; c < cols; c += 256 * 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + c);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      uint32_t out[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = __uint_as_float(u[j] << 16), hi = __uint_as_float(u[j] & 0xFFFF0000u);
        const uint32_t clo = e4m3_code((float)((double)lo / dsc));
        const uint32_t chi = e4m3_code((float)((double)hi / dsc));
        out[j >> 1] |= (clo | (chi << 8)) << (16 * (j & 1));
      }
      *reinterpret_cast<uint2*>(dst + c) = make_uint2(out[0], out[1]);
    }
    __syncthreads();                             // s_max is reused by the next row
  }
}

}  // namespace

hipError_t launch_quantize_fp8(const uint16_t* w, long long rows, int cols, uint8_t* q, float* scale,
                               hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const long long grid = rows < 65536 ? rows : 65536;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)grid), dim3(256), 0, st, w, rows, cols, q, scale);
  return hipGetLastError();
}

}  // namespace moe
