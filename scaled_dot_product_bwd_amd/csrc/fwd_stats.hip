// fwd_stats.hip -- statistics of the dense backward from what a forward pass
// saves: per (b, h, i) row the natural log-sum-exp of its scaled, masked scores
// and the output O.  delta = rowsum(dY * O) equals rowsum(P * dP) (O = P V, so
// dY . O = sum_j P_ij dY . V_j = sum_j P_ij dP_ij), which is how rlx-cpu
// `backward_dense_head_all` forms delta; the row's -lse2 = -lse log2 e is what
// the dK / dV and dQ kernels consume.  HBM-bound: dY and O are read once.
//
// A wave handles 4 rows at a time, 16 lanes per row, each lane 16 contiguous
// bytes of the row per step (coalesced), then a 16-lane sum.
#include "device_common.hpp"
#include "launch.hpp"

namespace attn {

template <typename T> __device__ __forceinline__ float dot16b(const T *a, const T *b);
template <> __device__ __forceinline__ float dot16b<bf16>(const bf16 *a, const bf16 *b) {
  const bf16x8 x = *reinterpret_cast<const bf16x8 *>(a), y = *reinterpret_cast<const bf16x8 *>(b);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = fmaf((float)x[e], (float)y[e], s);
  return s;
}
template <> __device__ __forceinline__ float dot16b<float>(const float *a, const float *b) {
  const f32x4 x = *reinterpret_cast<const f32x4 *>(a), y = *reinterpret_cast<const f32x4 *>(b);
  return fmaf(x[0], y[0], fmaf(x[1], y[1], fmaf(x[2], y[2], x[3] * y[3])));
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_fwd_stats(const DenseParams p, const float *lse,
                                                   const T *out, int64_t os0, int64_t os1,
                                                   int64_t os2) {
  constexpr int PER = 16 / sizeof(T);        // elements per lane step
  constexpr int STEPS = (D + 16 * PER - 1) / (16 * PER);
  const int lane = threadIdx.x & 63, sub = lane >> 4, l16 = lane & 15;
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  const int64_t wave_id = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int64_t row = wave_id * 4 + sub;  // (b * H + h) * Sq + i
  const bool valid = row < rows;
  const int64_t r = valid ? row : 0;
  const int i = (int)(r % p.Sq);
  const int64_t bh = r / p.Sq;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const T *g = (const T *)p.dy + b * p.dys[0] + (int64_t)i * p.dys[1] + h * p.dys[2];
  const T *o = out + b * os0 + (int64_t)i * os1 + h * os2;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < STEPS; ++k) {
    const int d0 = (k * 16 + l16) * PER;
    if (valid && d0 < D) s += dot16b<T>(g + d0, o + d0);
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (valid && l16 == 0) {
    const float L = lse[r];
    const bool empty = !(L > -INFINITY);  // a row that sees no key: P = 0, delta = 0
    p.st_delta[r] = empty ? 0.f : s;
    p.st_nls[r] = (empty ? -INFINITY : -L * kLog2e) * p.inv_scale_log2;
  }
}

hipError_t launch_fwd_stats(bool bf16_in, int D, const DenseParams &p, const float *lse,
                            const void *out, const int64_t *ostride, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  if (rows == 0) return hipSuccess;
  const int64_t waves = (rows + 3) / 4;
  const int blocks = (int)((waves + 3) / 4);
#define FWD_LAUNCH(TT, DD)                                                                     \
  hipLaunchKernelGGL((k_fwd_stats<TT, DD>), dim3(blocks), dim3(256), 0, stream, p, lse,        \
                     (const TT *)out, ostride[0], ostride[1], ostride[2])
  if (bf16_in) {
    if (D == 32) FWD_LAUNCH(bf16, 32); else if (D == 64) FWD_LAUNCH(bf16, 64); else FWD_LAUNCH(bf16, 128);
  } else {
    if (D == 32) FWD_LAUNCH(float, 32); else if (D == 64) FWD_LAUNCH(float, 64); else FWD_LAUNCH(float, 128);
  }
#undef FWD_LAUNCH
  return hipGetLastError();
}

}  // namespace attn
