// T == 1 decode step of the causal recurrence ("[Feature] LinearAttention layer
// for Keras", sections "Mathematical definition / Causal", "Masking / Causal",
// "Streaming State": token-by-token execution).  Per (b,h):
//   S' = S + phi(k) v^T,  Z' = Z + phi(k),  y = phi(q)^T S' / (phi(q)^T Z' + eps)
// and for a masked token S' = S, Z' = Z, y = 0.
//
// The step is pure HBM streaming: each unit reads and writes its fp32 state
// (Dk*Dv*4 bytes each way) and touches only 3 short vectors besides.  One
// 256-thread workgroup per unit; every thread issues all of its 16-byte state
// loads before doing any arithmetic so that a whole unit's state is in flight
// at once, then updates in registers, writes back and reduces the readout
// partials through LDS.
#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

template <typename DT>
__device__ __forceinline__ float load_elem(const DT* p, int i);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int i) {
  return bf16_bits_to_f32(p[i]);
}
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int i) {
  return p[i];
}

template <typename DT, int D, int FM, bool NORM>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  constexpr int C4 = D / 4;          // float4 columns per state row
  constexpr int RG = kThreads / C4;  // row groups
  constexpr int RPT = D / RG;        // rows per thread
  static_assert(RPT >= 1 && RG * RPT == D, "unsupported head size");
  __shared__ float fk[D], fq[D], zs[D];
  __shared__ float part[RG][D];
  __shared__ float den_s;

  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  const int b = u / a.H;
  const int c4 = tid % C4, rg = tid / C4;
  const float* S = a.s_in + (int64_t)u * D * D;
  float* So = a.s_out + (int64_t)u * D * D;

  f32x4_t sv[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) sv[r] = *(const f32x4_t*)(S + (rg + RG * r) * D + 4 * c4);

  const bool valid = a.mask ? (a.mask[b] != 0) : true;
  const DT* qp = (const DT*)a.q + (int64_t)u * D;
  const DT* kp = (const DT*)a.k + (int64_t)u * D;
  const DT* vp = (const DT*)a.v + (int64_t)u * D;
  float v4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v4[i] = valid ? load_elem<DT>(vp, 4 * c4 + i) : 0.f;
  if (tid < D) {
    const float kf = valid ? phi<FM>(load_elem<DT>(kp, tid), a.eps) : 0.f;
    fk[tid] = kf;
    fq[tid] = phi<FM>(load_elem<DT>(qp, tid), a.eps);
    if constexpr (NORM) zs[tid] = a.z_in[(int64_t)u * D + tid] + kf;
  }
  __syncthreads();

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int dk = rg + RG * r;
    const float f = fk[dk], g = fq[dk];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[r][i] = fmaf(f, v4[i], sv[r][i]);
      acc[i] = fmaf(g, sv[r][i], acc[i]);
    }
  }
  if (valid || So != S) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) *(f32x4_t*)(So + (rg + RG * r) * D + 4 * c4) = sv[r];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[rg][4 * c4 + i] = acc[i];
  if constexpr (NORM) {
    if (tid < 64) {
      float d = 0.f;
      for (int i = tid; i < D; i += 64) d = fmaf(fq[i], zs[i], d);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
      if (tid == 0) den_s = d + a.eps;
    }
    if (tid < D && (valid || a.z_out != a.z_in)) a.z_out[(int64_t)u * D + tid] = zs[tid];
  }
  __syncthreads();
  if (tid < D) {
    float y = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) y += part[g][tid];
    if constexpr (NORM) y = y / den_s;
    if (!valid) y = 0.f;
    DT* op = (DT*)a.out + (int64_t)u * D;
    if constexpr (sizeof(DT) == 2)
      ((uint16_t*)op)[tid] = (uint16_t)f32_to_bf16_bits(y);
    else
      ((float*)op)[tid] = y;
  }
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = 0.f;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(float* dst, const float* src, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    dst[i] = src[i];
}

template <typename DT, int D>
static hipError_t launch_d(int fm, int norm, const DecodeArgs& a, int units, hipStream_t st) {
  if (fm == kEluPlusOne) {
    if (norm)
      hipLaunchKernelGGL((decode_kernel<DT, D, kEluPlusOne, true>), dim3(units), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((decode_kernel<DT, D, kEluPlusOne, false>), dim3(units), dim3(kThreads), 0, st, a);
  } else {
    if (norm)
      hipLaunchKernelGGL((decode_kernel<DT, D, kReluEps, true>), dim3(units), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((decode_kernel<DT, D, kReluEps, false>), dim3(units), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

template <typename DT>
static hipError_t launch_dt(int D, int fm, int norm, const DecodeArgs& a, int units, hipStream_t st) {
  switch (D) {
    case 32: return launch_d<DT, 32>(fm, norm, a, units, st);
    case 64: return launch_d<DT, 64>(fm, norm, a, units, st);
    default: return launch_d<DT, 128>(fm, norm, a, units, st);
  }
}

hipError_t launch_decode(int bf16, int D, int fm, int norm, const DecodeArgs& a, int units,
                         hipStream_t st) {
  if (units <= 0) return hipSuccess;
  return bf16 ? launch_dt<uint16_t>(D, fm, norm, a, units, st)
              : launch_dt<float>(D, fm, norm, a, units, st);
}

static int grid_for(int64_t n) {
  int64_t g = (n + kThreads - 1) / kThreads;
  if (g > 65536) g = 65536;
  return (int)(g < 1 ? 1 : g);
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n)), dim3(kThreads), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_copy(float* dst, const float* src, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n)), dim3(kThreads), 0, st, dst, src, n);
  return hipGetLastError();
}

}  // namespace la
