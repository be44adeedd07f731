// k_quant.hip — block quantiser for the sym8 / int4 codecs.
//
// [QK] "鳴かぬなら、カスタムカーネル、ほととぎす" (qiita.com, john-rocky), section 6:
// weights are symmetric linear int8 with one scale per 32 consecutive K
// elements; section 3 and 7 describe the 4-bit variant.
// Per block: s = binary16(amax / qmax) (fp32 division, round to nearest even,
// saturated at 65504), then q = clamp(rint(w / s), -qmax, qmax) in fp32, q = 0
// when s is zero. The integer codes depend on every one of these fp32 steps,
// so none of them is reassociated or approximated.
#include "kernels.hpp"

namespace moe {

// One thread per block of 32 values.
template <int SCHEME>
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ w, int64_t nblocks,
                                                  uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblocks) return;
  constexpr int qmax = SCHEME == MOE_Q_SYM8 ? 127 : 7;
  float v[32];
  const float4* p = reinterpret_cast<const float4*>(w + i * 32);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float4 q = p[j];
    v[4 * j] = q.x; v[4 * j + 1] = q.y; v[4 * j + 2] = q.z; v[4 * j + 3] = q.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const float ratio = __fdiv_rn(amax, (float)qmax);
  uint16_t sb = __builtin_bit_cast(uint16_t, (_Float16)ratio);
  if ((sb & 0x7FFFu) == 0x7C00u) sb = (uint16_t)((sb & 0x8000u) | 0x7BFFu);
  scales[i] = sb;
  const float s = f16_bits_to_f32(sb);
  int q[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float t = 0.0f;
    if (s != 0.0f) {
      t = rintf(__fdiv_rn(v[j], s));
      t = fminf(fmaxf(t, (float)-qmax), (float)qmax);
    }
    q[j] = (int)t;
  }
  if constexpr (SCHEME == MOE_Q_SYM8) {
    uint32_t wd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      wd[j] = (uint32_t)(q[4 * j] & 0xFF) | ((uint32_t)(q[4 * j + 1] & 0xFF) << 8) |
              ((uint32_t)(q[4 * j + 2] & 0xFF) << 16) | ((uint32_t)(q[4 * j + 3] & 0xFF) << 24);
    uint4* out = reinterpret_cast<uint4*>(codes + i * 32);
    out[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    out[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
  } else {
    uint32_t wd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t acc = 0;
#pragma unroll
      for (int n = 0; n < 8; ++n) acc |= (uint32_t)(q[8 * j + n] & 0xF) << (4 * n);
      wd[j] = acc;
    }
    *reinterpret_cast<uint4*>(codes + i * 16) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
}

hipError_t launch_quantize(const float* w, int64_t rows, int K, int scheme, uint8_t* codes, uint16_t* scales,
                           hipStream_t s) {
  const int64_t nblocks = rows * (K / 32);
  if (nblocks == 0) return hipSuccess;
  dim3 grid((unsigned)((nblocks + 255) / 256));
  if (scheme == MOE_Q_SYM8) MOE_LAUNCH(MOE_KERNEL_QUANTIZE, k_quantize<MOE_Q_SYM8>, grid, dim3(256), 0, s, w, nblocks, codes, scales);
  else MOE_LAUNCH(MOE_KERNEL_QUANTIZE, k_quantize<MOE_Q_INT4>, grid, dim3(256), 0, s, w, nblocks, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
