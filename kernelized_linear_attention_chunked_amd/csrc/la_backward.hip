// Elementwise and scan kernels of the causal backward pass (gradients of the
// normalized causal recurrence; the Keras proposal asks for recurrent/parallel
// gradient parity and float64 numerical-gradient checks, "Stability" and
// "Acceptance").  With phi_q = phi(q), phi_k = phi(k) (0 at invalid tokens),
// z_i = z_0 + sum_{j<=i} phi_k_j and den_i = phi_q_i . z_i + eps:
//   dnum_i = m_i dy_i / den_i,   dden_i = -m_i (dy_i . num_i) / den_i^2  (normalized)
//   dnum_i = m_i dy_i,           dden_i = 0                              (otherwise)
// and since dy_i . num_i = phi_q_i . (S_i dy_i), dden_i = -(phi_q_i . qa_i) / den_i
// with qa_i = S_i dnum_i, the first recurrence's fp32 output.  den_i itself is
// formed here in fp32 from the prefix sums z_i, so that the terms of
// dphi_q_i = qa_i + z_i dden_i, which nearly cancel, cancel to fp32 precision.
//   dphi_q_i = S_i dnum_i + z_i dden_i
//   dphi_k_j = sum_{i>=j} phi_q_i (v_j . dnum_i) + dS_T v_j + [dz_T + sum_{i>=j} phi_q_i dden_i]
//   dv_j     = sum_{i>=j} dnum_i (phi_q_i . phi_k_j) + dS_T^T phi_k_j
//   dS_0 = dS_T + sum_i phi_q_i dnum_i^T,   dz_0 = dz_T + sum_i phi_q_i dden_i.
// The three sums of products are linear-rule recurrences (la_gated.hip, run by
// the front end, the last two in reversed time); the kernels here prepare their
// inputs, form the prefix sums and combine the results.
#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

template <typename IT>
__device__ __forceinline__ float ld_io(const IT* p, int64_t i) {
  if constexpr (sizeof(IT) == 2) return Io<IT>::to_f32(((const uint16_t*)p)[i]);
  else return ((const float*)p)[i];
}
template <typename IT>
__device__ __forceinline__ void st_io(IT* p, int64_t i, float x) {
  if constexpr (std::is_same_v<IT, uint16_t>) ((uint16_t*)p)[i] = (uint16_t)f32_to_bf16_bits(x);
  else p[i] = (IT)x;
}
// derivative of phi: elu(x)+1 -> 1 (x > 0) or exp(x); relu(x)+eps -> 1 (x > 0) or 0
__device__ __forceinline__ float dphi(float x, int fm) {
  if (fm == kEluPlusOne) return x > 0.f ? 1.f : __expf(x);
  return x > 0.f ? 1.f : 0.f;
}

// phi(q), phi(k) (0 at invalid tokens), v (0 at invalid tokens) as fp32.
template <typename IT, int FM>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(BwdArgs a) {
  const int64_t HD = (int64_t)a.H * a.D;
  const int64_t n = (int64_t)a.B * a.T * HD;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int64_t bt = i / HD;
    const bool m = a.mask ? a.mask[bt] != 0 : true;
    a.fq[i] = phi<FM>(ld_io((const IT*)a.q, i), a.eps);
    a.fk[i] = m ? phi<FM>(ld_io((const IT*)a.k, i), a.eps) : 0.f;
    a.v32[i] = m ? ld_io((const IT*)a.v, i) : 0.f;
  }
}

// Running sums over T per (b, h, d): out[t] = init + sum x[t'] w[t'] over t' <= t
// (forward) or t' >= t (reverse); w (B,T,H) may be null (1).  One workgroup
// per (b, h): thread (segment, d) sums its segment, the segment offsets come
// through LDS, then a second sweep writes the running sums (independent loads,
// unrolled; x and out never alias).  total (B,H,D), if given, receives init +
// the sum over all t.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void bwd_scan_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ w,
                                                                const float* __restrict__ init,
                                                                float* __restrict__ out, float* __restrict__ total,
                                                                int T, int H, int D, int reverse) {
  __shared__ float part[kScanThreads];
  const int u = blockIdx.x, b = u / H, h = u % H;
  const int tid = threadIdx.x, d = tid % D, sg = tid / D, nseg = kScanThreads / D;
  const int len = (T + nseg - 1) / nseg;
  const int t0 = min(T, sg * len), t1 = min(T, t0 + len);
  auto at = [&](int t) { return (((int64_t)b * T + t) * H + h) * D + d; };
  auto wt = [&](int t) { return w ? w[((int64_t)b * T + t) * H + h] : 1.f; };
  float s = 0.f;
#pragma unroll 8
  for (int t = t0; t < t1; ++t) s += x[at(t)] * wt(t);
  part[tid] = s;
  __syncthreads();
  float run = init ? init[(int64_t)u * D + d] : 0.f;
  for (int g = 0; g < nseg; ++g) {
    const bool before = reverse ? g > sg : g < sg;
    if (before) run += part[g * D + d];
  }
  if (total && sg == 0) {
    float all = init ? init[(int64_t)u * D + d] : 0.f;
    for (int g = 0; g < nseg; ++g) all += part[g * D + d];
    total[(int64_t)u * D + d] = all;
  }
  if (!reverse) {
#pragma unroll 8
    for (int t = t0; t < t1; ++t) {
      run += x[at(t)] * wt(t);
      out[at(t)] = run;
    }
  } else {
#pragma unroll 8
    for (int t = t1 - 1; t >= t0; --t) {
      run += x[at(t)] * wt(t);
      out[at(t)] = run;
    }
  }
}

// den (normalized: phi_q . z + eps in fp32) and dnum
// per token: one wave per (b, t, h).
template <typename IT>
__global__ __launch_bounds__(kThreads) void bwd_dnum_kernel(BwdArgs a) {
  const int64_t ntok = (int64_t)a.B * a.T * a.H;
  const int64_t tk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (tk >= ntok) return;  // whole waves
  const int l = threadIdx.x & 63;
  const int64_t bt = tk / a.H;
  const bool m = a.mask ? a.mask[bt] != 0 : true;
  const int64_t base = tk * a.D;
  float rden = 1.f;
  if (a.den) {
    float dot = 0.f;
    for (int d = l; d < a.D; d += 64) dot += a.fq[base + d] * a.zc[base + d];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
    const float den = dot + a.eps;
    if (l == 0) a.den[tk] = den;
    rden = 1.f / den;
  }
  for (int d = l; d < a.D; d += 64) {
    a.dnum[base + d] = m ? ld_io((const IT*)a.dy, base + d) * rden : 0.f;
  }
}

// dden_i = -m_i (phi_q_i . qa_i) / den_i (normalized): one wave per (b, t, h).
__global__ __launch_bounds__(kThreads) void bwd_dden_kernel(BwdArgs a) {
  const int64_t ntok = (int64_t)a.B * a.T * a.H;
  const int64_t tk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (tk >= ntok) return;  // whole waves
  const int l = threadIdx.x & 63;
  const int64_t bt = tk / a.H;
  const bool m = a.mask ? a.mask[bt] != 0 : true;
  const int64_t base = tk * a.D;
  float dot = 0.f;
  for (int d = l; d < a.D; d += 64) dot += a.fq[base + d] * a.qa[base + d];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
  if (l == 0) a.dden[tk] = m ? -dot / a.den[tk] : 0.f;
}

// dq, dk, dv from the recurrences' outputs: dq = (A + z dden) phi'(q),
// dk = (C + R) phi'(k), dv = Dv, 0 at invalid tokens.
template <typename IT>
__global__ __launch_bounds__(kThreads) void bwd_finish_kernel(BwdArgs a) {
  const int64_t HD = (int64_t)a.H * a.D;
  const int64_t n = (int64_t)a.B * a.T * HD;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int64_t bt = i / HD, r = i % HD;
    const bool m = a.mask ? a.mask[bt] != 0 : true;
    float gq = 0.f, gk = 0.f, gv = 0.f;
    if (m) {
      float pq = a.qa[i], pk = a.kc[i];
      if (a.zc) pq += a.zc[i] * a.dden[bt * a.H + r / a.D];
      if (a.rs) pk += a.rs[i];
      gq = pq * dphi(ld_io((const IT*)a.q, i), a.fm);
      gk = pk * dphi(ld_io((const IT*)a.k, i), a.fm);
      gv = a.vd[i];
    }
    st_io((IT*)a.dq, i, gq);
    st_io((IT*)a.dk, i, gk);
    st_io((IT*)a.dv, i, gv);
  }
}

// out[u][c][r] = in[u][r][c] for U square D x D matrices
__global__ __launch_bounds__(kThreads) void bwd_transpose_kernel(const float* in, float* out, int64_t U, int D) {
  const int64_t n = U * D * D;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int64_t u = i / ((int64_t)D * D), e = i % ((int64_t)D * D);
    const int r = (int)(e / D), c = (int)(e % D);
    out[u * D * D + (int64_t)c * D + r] = in[i];
  }
}

static int grid_of(int64_t n) {
  int64_t g = (n + kThreads - 1) / kThreads;
  if (g > 65536) g = 65536;
  return (int)(g < 1 ? 1 : g);
}

template <typename IT>
static void launch_prep_t(const BwdArgs& a, hipStream_t st) {
  const int grid = grid_of((int64_t)a.B * a.T * a.H * a.D);
  if (a.fm == kEluPlusOne)
    hipLaunchKernelGGL((bwd_prep_kernel<IT, kEluPlusOne>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_prep_kernel<IT, kReluEps>), dim3(grid), dim3(kThreads), 0, st, a);
}

hipError_t launch_bwd_prep(int io, const BwdArgs& a, hipStream_t st) {
  switch (io) {
    case kIoBF16: launch_prep_t<uint16_t>(a, st); break;
    case kIoF16: launch_prep_t<f16_t>(a, st); break;
    default: launch_prep_t<float>(a, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_scan(const float* x, const float* w, const float* init, float* out, float* total, int U,
                           int T, int H, int D, int reverse, hipStream_t st) {
  if (U <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_scan_kernel, dim3(U), dim3(kScanThreads), 0, st, x, w, init, out, total, T, H, D,
                     reverse);
  return hipGetLastError();
}

hipError_t launch_bwd_dnum(int io, const BwdArgs& a, hipStream_t st) {
  const int64_t ntok = (int64_t)a.B * a.T * a.H;
  const int64_t grid = (ntok + (kThreads / 64) - 1) / (kThreads / 64);
  switch (io) {
    case kIoBF16: hipLaunchKernelGGL(bwd_dnum_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, st, a); break;
    case kIoF16: hipLaunchKernelGGL(bwd_dnum_kernel<f16_t>, dim3(grid), dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL(bwd_dnum_kernel<float>, dim3(grid), dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dden(const BwdArgs& a, hipStream_t st) {
  const int64_t ntok = (int64_t)a.B * a.T * a.H;
  const int64_t grid = (ntok + (kThreads / 64) - 1) / (kThreads / 64);
  hipLaunchKernelGGL(bwd_dden_kernel, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_finish(int io, const BwdArgs& a, hipStream_t st) {
  const int grid = grid_of((int64_t)a.B * a.T * a.H * a.D);
  switch (io) {
    case kIoBF16: hipLaunchKernelGGL(bwd_finish_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, st, a); break;
    case kIoF16: hipLaunchKernelGGL(bwd_finish_kernel<f16_t>, dim3(grid), dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL(bwd_finish_kernel<float>, dim3(grid), dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_transpose(const float* in, float* out, int64_t U, int D, hipStream_t st) {
  if (U <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_transpose_kernel, dim3(grid_of(U * D * D)), dim3(kThreads), 0, st, in, out, U, D);
  return hipGetLastError();
}

}  // namespace la
