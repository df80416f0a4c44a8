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

// four consecutive elements from element i (i % 4 == 0; the buffers are 16-byte aligned)
template <typename IT>
__device__ __forceinline__ f32x4_t ld4_io(const IT* p, int64_t i) {
  if constexpr (sizeof(IT) == 2) {
    const u32x2_t w = *(const u32x2_t*)((const uint16_t*)p + i);
    return f32x4_t{Io<IT>::to_f32(w[0] & 0xffffu), Io<IT>::to_f32(w[0] >> 16), Io<IT>::to_f32(w[1] & 0xffffu),
                   Io<IT>::to_f32(w[1] >> 16)};
  } else {
    return *(const f32x4_t*)((const float*)p + i);
  }
}
template <typename IT>
__device__ __forceinline__ void st4_io(IT* p, int64_t i, const f32x4_t& x) {
  store4(p + i, x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ f32x4_t ld4(const float* p, int64_t i) { return *(const f32x4_t*)(p + i); }
__device__ __forceinline__ void st4(float* p, int64_t i, const f32x4_t& x) { *(f32x4_t*)(p + i) = x; }
// derivative of phi: elu(x)+1 -> 1 (x > 0) or exp(x); relu(x)+eps -> 1 (x > 0) or 0
__device__ __forceinline__ float dphi(float x, int fm) {
  if (fm == kEluPlusOne) return x > 0.f ? 1.f : __expf(x);
  return x > 0.f ? 1.f : 0.f;
}

// phi(q), phi(k) (0 at invalid tokens), v (0 at invalid tokens) as fp32; four
// consecutive elements per thread (D % 4 == 0: one token-head each).
template <typename IT, int FM>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(BwdArgs a) {
  const int64_t HD = (int64_t)a.H * a.D;
  const int64_t n4 = (int64_t)a.B * a.T * HD / 4;
  for (int64_t i4 = (int64_t)blockIdx.x * kThreads + threadIdx.x; i4 < n4; i4 += (int64_t)gridDim.x * kThreads) {
    const int64_t i = 4 * i4, bt = i / HD;
    const bool m = a.mask ? a.mask[bt] != 0 : true;
    const f32x4_t q = ld4_io((const IT*)a.q, i), k = ld4_io((const IT*)a.k, i), v = ld4_io((const IT*)a.v, i);
    f32x4_t fq, fk, vv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fq[e] = phi<FM>(q[e], a.eps);
      fk[e] = m ? phi<FM>(k[e], a.eps) : 0.f;
      vv[e] = m ? v[e] : 0.f;
    }
    st4(a.fq, i, fq);
    st4(a.fk, i, fk);
    st4(a.v32, i, vv);
  }
}

// Running sums over T per (b, h, d): out[t] = init + sum x[t'] w[t'] over t' <= t
// (forward) or t' >= t (reverse); w (B,T,H) may be null (1).  The columns d
// are independent: workgroup (b, h, part) takes DC = D / dsplit of them, and
// its thread (segment, d) sums its segment of T, the segment offsets come
// through LDS, then a second sweep writes the running sums (independent loads,
// unrolled; x and out never alias).  total (B,H,D), if given, receives init +
// the sum over all t.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void bwd_scan_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ w,
                                                                const float* __restrict__ init,
                                                                float* __restrict__ out, float* __restrict__ total,
                                                                int T, int H, int D, int reverse, int dsplit) {
  __shared__ float part[kScanThreads];
  const int u = blockIdx.x / dsplit, b = u / H, h = u % H;
  const int DC = D / dsplit;
  const int tid = threadIdx.x, dc = tid % DC, d = (blockIdx.x % dsplit) * DC + dc, sg = tid / DC,
            nseg = kScanThreads / DC;
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
    if (before) run += part[g * DC + dc];
  }
  if (total && sg == 0) {
    float all = init ? init[(int64_t)u * D + d] : 0.f;
    for (int g = 0; g < nseg; ++g) all += part[g * DC + dc];
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

// Per-token dot products over D: D/4 lanes per (b, t, h), four consecutive
// elements each, summed by xor shuffles inside the lane group (D/4 divides 64,
// so a group never straddles a wave and whole groups exit together).
__device__ __forceinline__ float group_sum(float x, int lpt) {
  for (int off = lpt >> 1; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// den (normalized: phi_q . z + eps in fp32) and dnum.
template <typename IT>
__global__ __launch_bounds__(kThreads) void bwd_dnum_kernel(BwdArgs a) {
  const int lpt = a.D >> 2;
  const int64_t ntok = (int64_t)a.B * a.T * a.H;
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t tk = g / lpt;
  if (tk >= ntok) return;
  const int64_t bt = tk / a.H;
  const bool m = a.mask ? a.mask[bt] != 0 : true;
  const int64_t i = tk * a.D + 4 * (g % lpt);
  float rden = 1.f;
  if (a.den) {
    const f32x4_t fq = ld4(a.fq, i), z = ld4(a.zc, i);
    const float den = group_sum(fq[0] * z[0] + fq[1] * z[1] + fq[2] * z[2] + fq[3] * z[3], lpt) + a.eps;
    if (g % lpt == 0) a.den[tk] = den;
    rden = 1.f / den;
  }
  const f32x4_t dy = ld4_io((const IT*)a.dy, i);
  f32x4_t r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = m ? dy[e] * rden : 0.f;
  st4(a.dnum, i, r);
}

// dden_i = -m_i (phi_q_i . qa_i) / den_i (normalized).
__global__ __launch_bounds__(kThreads) void bwd_dden_kernel(BwdArgs a) {
  const int lpt = a.D >> 2;
  const int64_t ntok = (int64_t)a.B * a.T * a.H;
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t tk = g / lpt;
  if (tk >= ntok) return;
  const int64_t bt = tk / a.H;
  const bool m = a.mask ? a.mask[bt] != 0 : true;
  const int64_t i = tk * a.D + 4 * (g % lpt);
  const f32x4_t fq = ld4(a.fq, i), qa = ld4(a.qa, i);
  const float dot = group_sum(fq[0] * qa[0] + fq[1] * qa[1] + fq[2] * qa[2] + fq[3] * qa[3], lpt);
  if (g % lpt == 0) a.dden[tk] = m ? -dot / a.den[tk] : 0.f;
}

// dq, dk, dv from the recurrences' outputs: dq = (A + z dden) phi'(q),
// dk = (C + R) phi'(k), dv = Dv, 0 at invalid tokens.
template <typename IT>
__global__ __launch_bounds__(kThreads) void bwd_finish_kernel(BwdArgs a) {
  const int64_t HD = (int64_t)a.H * a.D;
  const int64_t n4 = (int64_t)a.B * a.T * HD / 4;
  for (int64_t i4 = (int64_t)blockIdx.x * kThreads + threadIdx.x; i4 < n4; i4 += (int64_t)gridDim.x * kThreads) {
    const int64_t i = 4 * i4, bt = i / HD, r = i % HD;
    const bool m = a.mask ? a.mask[bt] != 0 : true;
    f32x4_t gq = {0.f, 0.f, 0.f, 0.f}, gk = gq, gv = gq;
    if (m) {
      f32x4_t pq = ld4(a.qa, i), pk = ld4(a.kc, i);
      if (a.zc) {
        const float dd = a.dden[bt * a.H + r / a.D];
        const f32x4_t z = ld4(a.zc, i);
#pragma unroll
        for (int e = 0; e < 4; ++e) pq[e] += z[e] * dd;
      }
      if (a.rs) {
        const f32x4_t rr = ld4(a.rs, i);
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] += rr[e];
      }
      const f32x4_t q = ld4_io((const IT*)a.q, i), k = ld4_io((const IT*)a.k, i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gq[e] = pq[e] * dphi(q[e], a.fm);
        gk[e] = pk[e] * dphi(k[e], a.fm);
      }
      gv = ld4(a.vd, i);
    }
    st4_io((IT*)a.dq, i, gq);
    st4_io((IT*)a.dk, i, gk);
    st4_io((IT*)a.dv, i, gv);
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
  const int grid = grid_of((int64_t)a.B * a.T * a.H * a.D / 4);
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
  // columns split over workgroups until the grid covers the 256 CUs, keeping
  // at least 16 columns (64-byte row pieces) per workgroup
  int dsplit = 1;
  while ((int64_t)U * dsplit < 256 && D / (2 * dsplit) >= 16) dsplit *= 2;
  hipLaunchKernelGGL(bwd_scan_kernel, dim3(U * dsplit), dim3(kScanThreads), 0, st, x, w, init, out, total, T, H,
                     D, reverse, dsplit);
  return hipGetLastError();
}

// one thread per four elements of the (B, T, H, D) buffers
static int64_t dot_grid(const BwdArgs& a) {
  const int64_t n4 = (int64_t)a.B * a.T * a.H * (a.D / 4);
  return (n4 + kThreads - 1) / kThreads;
}

hipError_t launch_bwd_dnum(int io, const BwdArgs& a, hipStream_t st) {
  const int64_t grid = dot_grid(a);
  switch (io) {
    case kIoBF16: hipLaunchKernelGGL(bwd_dnum_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, st, a); break;
    case kIoF16: hipLaunchKernelGGL(bwd_dnum_kernel<f16_t>, dim3(grid), dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL(bwd_dnum_kernel<float>, dim3(grid), dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dden(const BwdArgs& a, hipStream_t st) {
  const int64_t grid = dot_grid(a);
  hipLaunchKernelGGL(bwd_dden_kernel, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_finish(int io, const BwdArgs& a, hipStream_t st) {
  const int grid = grid_of((int64_t)a.B * a.T * a.H * a.D / 4);
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
