// T == 1 decode step of the causal recurrence ("[Feature] LinearAttention layer
// for Keras", sections "Mathematical definition / Causal", "Masking / Causal",
// "Streaming State": token-by-token execution).  Per (b,h):
//   S' = S + phi(k) v^T,  Z' = Z + phi(k),  y = phi(q)^T S' / (phi(q)^T Z' + eps)
// and for a masked token S' = S, Z' = Z, y = 0.
//
// The step is pure HBM streaming: each unit reads and writes its fp32 state
// (Dk*Dv*4 bytes each way) and touches only 3 short vectors besides.  256
// threads per unit, two units per workgroup; every thread issues all of its
// 16-byte state loads before doing any arithmetic so that a whole unit's state
// is in flight at once, then updates in registers, writes back and reduces the
// readout partials through LDS.
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
__device__ __forceinline__ float load_elem<f16_t>(const f16_t* p, int i) {
  return (float)p[i];
}
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int i) {
  return p[i];
}

// Two units per 512-thread workgroup: measured on the streaming workload's
// shape (8192 units of 128x128), this and non-temporal state accesses move the
// kernel from 5.1 to 5.9 TB/s.
constexpr int kDecodeUnits = 2;
constexpr int kDecodeThreads = kDecodeUnits * kThreads;

// DK, DV: head sizes of q/k and v; TPU threads per unit, UPB units per
// workgroup.  Thread (c4, rg) holds columns 4*c4 .. 4*c4+3 of state rows
// rg + RG*r.
template <typename DT, int DK, int DV, int FM, bool NORM, bool NTMP, int TPU = kThreads, int UPB = kDecodeUnits>
__global__ __launch_bounds__(TPU * UPB) void decode_kernel(DecodeArgs a) {
  constexpr int C4 = DV / 4;         // float4 columns per state row
  constexpr int RG = TPU / C4;       // row groups
  constexpr int RPT = DK / RG;       // rows per thread
  static_assert(RPT >= 1 && RG * RPT == DK && TPU >= DK && TPU >= DV && TPU >= 64, "unsupported head size");
  __shared__ float fk[UPB][DK], fq[UPB][DK], zs[UPB][DK];
  __shared__ float part[UPB][RG][DV];
  __shared__ float den_s[UPB];

  const int ul = threadIdx.x / TPU;  // unit slot in the workgroup
  const int tid = threadIdx.x % TPU;
  const int u = blockIdx.x * UPB + ul;
  const bool live = u < a.units;  // the last workgroup may hold one unit only
  const int b = u / a.H;
  const int c4 = tid % C4, rg = tid / C4;
  const float* S = a.s_in + (int64_t)u * DK * DV;
  float* So = a.s_out + (int64_t)u * DK * DV;

  f32x4_t sv[RPT];
  if (live) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const f32x4_t* p = (const f32x4_t*)(S + (rg + RG * r) * DV + 4 * c4);
      sv[r] = NTMP ? __builtin_nontemporal_load(p) : *p;
    }
  }
  const bool valid = live && (a.mask ? (a.mask[b] != 0) : true);
  const DT* qp = (const DT*)a.q + (int64_t)u * DK;
  const DT* kp = (const DT*)a.k + (int64_t)u * DK;
  const DT* vp = (const DT*)a.v + (int64_t)u * DV;
  float v4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v4[i] = valid ? load_elem<DT>(vp, 4 * c4 + i) : 0.f;
  if (live && tid < DK) {
    const float kf = valid ? phi<FM>(load_elem<DT>(kp, tid), a.eps) : 0.f;
    fk[ul][tid] = kf;
    fq[ul][tid] = phi<FM>(load_elem<DT>(qp, tid), a.eps);
    if constexpr (NORM) zs[ul][tid] = a.z_in[(int64_t)u * DK + tid] + kf;
  }
  __syncthreads();
  if (live) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int dk = rg + RG * r;
      const float f = fk[ul][dk], g = fq[ul][dk];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[r][i] = fmaf(f, v4[i], sv[r][i]);
        acc[i] = fmaf(g, sv[r][i], acc[i]);
      }
    }
    if (valid || So != S) {
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        f32x4_t* p = (f32x4_t*)(So + (rg + RG * r) * DV + 4 * c4);
        if constexpr (NTMP)
          __builtin_nontemporal_store(sv[r], p);
        else
          *p = sv[r];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) part[ul][rg][4 * c4 + i] = acc[i];
    if constexpr (NORM) {
      if (tid < 64) {
        float d = 0.f;
        for (int i = tid; i < DK; i += 64) d = fmaf(fq[ul][i], zs[ul][i], d);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
        if (tid == 0) den_s[ul] = d + a.eps;
      }
      if (tid < DK && (valid || a.z_out != a.z_in)) a.z_out[(int64_t)u * DK + tid] = zs[ul][tid];
    }
  }
  __syncthreads();
  if (live && tid < DV) {
    float y = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) y += part[ul][g][tid];
    if constexpr (NORM) y = y / den_s[ul];
    if (!valid) y = 0.f;
    DT* op = (DT*)a.out + (int64_t)u * DV;
    if constexpr (std::is_same_v<DT, uint16_t>)
      op[tid] = (uint16_t)f32_to_bf16_bits(y);
    else
      op[tid] = (DT)y;
  }
}

// T == 1 step of the gated recurrence with grouped query heads (the
// LinearAttention operator page, "gated" / "linear" update rules, one token):
// per (b, kv head j)
//   S' = exp(g) S + k v^T,   o_h = scale q_h^T S'   for the G query heads of j.
// The same streaming layout as decode_kernel: a thread owns RPT rows of four
// consecutive state columns, issues all of its state loads first, updates in
// registers, writes back, and keeps partial readouts of every query head; the
// row groups are summed through LDS.  q and k are staged in LDS as fp32.
template <typename DT, int D, int G, bool NTMP, bool PD, bool MP, int TPU = kThreads, int UPB = kDecodeUnits>
__global__ __launch_bounds__(TPU * UPB) void gated_step_kernel(GatedStepArgs a) {
  // G query heads per readout pass; MP: a.heads / G passes (a kv head with
  // more heads, or a head count that is not a power of two), else one
  constexpr int C4 = D / 4;          // float4 columns per state row
  constexpr int RG = TPU / C4;  // row groups
  constexpr int RPT = D / RG;        // rows per thread
  static_assert(RPT >= 1 && RG * RPT == D && C4 <= 32, "unsupported head size");
  __shared__ float fk[UPB][D], fq[UPB][G][D], fe[UPB][PD ? D : 1];
  __shared__ float part[UPB][G][RG][D];

  const int ul = threadIdx.x / TPU;  // unit slot in the workgroup
  const int tid = threadIdx.x % TPU;
  const int u = blockIdx.x * UPB + ul;
  const bool live = u < a.units;  // the last workgroup may hold one unit only
  const int b = u / a.Hkv, j = u % a.Hkv;
  const int c4 = tid % C4, rg = tid / C4;
  const int64_t SE = (int64_t)D * D;
  const int NPASS = MP ? a.heads / G : 1;
  const int GT = G * NPASS;  // query heads of the kv head

  f32x4_t sv[RPT];
  if (live && a.s_in) {
    const float* S = a.s_in + (int64_t)u * SE;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const f32x4_t* p = (const f32x4_t*)(S + (rg + RG * r) * D + 4 * c4);
      sv[r] = NTMP ? __builtin_nontemporal_load(p) : *p;
    }
  } else {
#pragma unroll
    for (int r = 0; r < RPT; ++r) sv[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int QW = a.Hkv * GT * D;  // query row width
  // row of batch b in the token tensors, and (row, kv head) index
  const int64_t br = (int64_t)b * (a.batch_rows > 1 ? a.batch_rows : 1), uh = br * a.Hkv + j;
  const DT* qp = (const DT*)a.q + br * QW + (int64_t)j * GT * D;
  const DT* kp = (const DT*)a.k + uh * D;
  const DT* vp = (const DT*)a.v + uh * D;
  // fp32 copies of the query rows of pass p
  auto load_q = [&](int p) {
    const DT* qpp = qp + (int64_t)p * G * D;
    for (int i = tid; i < G * D; i += TPU) fq[ul][i / D][i % D] = load_elem<DT>(qpp, i);
  };
  float v4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v4[i] = live ? load_elem<DT>(vp, 4 * c4 + i) : 0.f;
  const float e = (live && a.decay && !PD) ? __expf(load_elem<DT>((const DT*)a.decay, uh)) : 1.f;
  if (live) {
    for (int i = tid; i < D; i += TPU) fk[ul][i] = load_elem<DT>(kp, i);
    if constexpr (PD)  // per-key-dim decay: row dk of S scales by exp(g[dk])
      for (int i = tid; i < D; i += TPU) fe[ul][i] = __expf(load_elem<DT>((const DT*)a.decay + uh * D, i));
    load_q(0);
  }
  __syncthreads();
  for (int p = 0; p < NPASS; ++p) {
    if (p > 0) {
      // the previous pass read fq before its last barrier
      if (live) load_q(p);
      __syncthreads();
    }
    if (live) {
      float acc[G][4];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[h][i] = 0.f;
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int dk = rg + RG * r;
        if (p == 0) {
          const float f = fk[ul][dk];
          const float er = PD ? fe[ul][dk] : e;
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[r][i] = fmaf(f, v4[i], er * sv[r][i]);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float g = fq[ul][h][dk];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[h][i] = fmaf(g, sv[r][i], acc[h][i]);
        }
      }
      if (p == 0) {
        float* So = a.s_out + (int64_t)u * SE;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          f32x4_t* ptr = (f32x4_t*)(So + (rg + RG * r) * D + 4 * c4);
          if constexpr (NTMP)
            __builtin_nontemporal_store(sv[r], ptr);
          else
            *ptr = sv[r];
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[ul][h][rg][4 * c4 + i] = acc[h][i];
    }
    __syncthreads();
    if (live) {
      DT* op = (DT*)a.out + br * QW + (int64_t)j * GT * D + (int64_t)p * G * D;
      for (int i = tid; i < G * D; i += TPU) {
        const int h = i / D, d = i % D;
        float y = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g) y += part[ul][h][g][d];
        y *= a.scale;
        if constexpr (std::is_same_v<DT, uint16_t>)
          op[i] = (uint16_t)f32_to_bf16_bits(y);
        else
          op[i] = (DT)y;
      }
    }
  }
}

// T == 1 step of the delta rules (the LinearAttention operator page, update
// rules "delta" and "gated_delta", one token): per (b, kv head j)
//   S' = E S,  u = beta (v - S'^T k),  S'' = S' + k u^T,  o_h = scale q_h^T S''
// with E = I, exp(g) or diag(exp(g)) (DK 0, 1, 2).  The gated step's layout:
// a thread owns RPT rows of four consecutive state columns and keeps them in
// registers throughout.  Two sums over the rows go through LDS in turn: S'^T k
// (then u, one value per column), and after the rank-1 update q_h^T S''.  One
// read and one write of the state, as for the gated step.
template <typename DT, int D, int G, bool NTMP, int DK, bool MP, int TPU = kThreads, int UPB = kDecodeUnits>
__global__ __launch_bounds__(TPU * UPB) void delta_step_kernel(GatedStepArgs a) {
  // G query heads per readout pass; MP: a.heads / G passes, else one
  constexpr int C4 = D / 4;          // float4 columns per state row
  constexpr int RG = TPU / C4;  // row groups
  constexpr int RPT = D / RG;        // rows per thread
  static_assert(RPT >= 1 && RG * RPT == D && C4 <= 32, "unsupported head size");
  __shared__ float fk[UPB][D], fq[UPB][G][D], fe[UPB][DK == 2 ? D : 1];
  __shared__ float fu[UPB][D];
  __shared__ float part[UPB][G][RG][D];

  const int ul = threadIdx.x / TPU;  // unit slot in the workgroup
  const int tid = threadIdx.x % TPU;
  const int u = blockIdx.x * UPB + ul;
  const bool live = u < a.units;  // the last workgroup may hold one unit only
  const int b = u / a.Hkv, j = u % a.Hkv;
  const int c4 = tid % C4, rg = tid / C4;
  const int64_t SE = (int64_t)D * D;
  const int NPASS = MP ? a.heads / G : 1;
  const int GT = G * NPASS;  // query heads of the kv head

  f32x4_t sv[RPT];
  if (live && a.s_in) {
    const float* S = a.s_in + (int64_t)u * SE;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const f32x4_t* p = (const f32x4_t*)(S + (rg + RG * r) * D + 4 * c4);
      sv[r] = NTMP ? __builtin_nontemporal_load(p) : *p;
    }
  } else {
#pragma unroll
    for (int r = 0; r < RPT; ++r) sv[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int QW = a.Hkv * GT * D;  // query row width
  // row of batch b in the token tensors, and (row, kv head) index
  const int64_t br = (int64_t)b * (a.batch_rows > 1 ? a.batch_rows : 1), uh = br * a.Hkv + j;
  const DT* qp = (const DT*)a.q + br * QW + (int64_t)j * GT * D;
  const DT* kp = (const DT*)a.k + uh * D;
  const DT* vp = (const DT*)a.v + uh * D;
  auto load_q = [&](int p) {
    const DT* qpp = qp + (int64_t)p * G * D;
    for (int i = tid; i < G * D; i += TPU) fq[ul][i / D][i % D] = load_elem<DT>(qpp, i);
  };
  const float e = (live && DK == 1) ? __expf(load_elem<DT>((const DT*)a.decay, uh)) : 1.f;
  const float be = live ? load_elem<DT>((const DT*)a.beta, br * a.beta_heads + (a.beta_heads > 1 ? j : 0)) : 0.f;
  const float vc = (live && tid < D) ? load_elem<DT>(vp, tid) : 0.f;  // v of column tid
  if (live) {
    for (int i = tid; i < D; i += TPU) fk[ul][i] = load_elem<DT>(kp, i);
    if constexpr (DK == 2)  // per-key-dim decay: row dk of S scales by exp(g[dk])
      for (int i = tid; i < D; i += TPU) fe[ul][i] = __expf(load_elem<DT>((const DT*)a.decay + uh * D, i));
    load_q(0);
  }
  __syncthreads();
  // S' = E S, and the thread's part of S'^T k
  if (live) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int dk = rg + RG * r;
      const float er = DK == 2 ? fe[ul][dk] : e;
      const float f = fk[ul][dk];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[r][i] *= er;
        acc[i] = fmaf(f, sv[r][i], acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) part[ul][0][rg][4 * c4 + i] = acc[i];
  }
  __syncthreads();
  // u = beta (v - S'^T k), one column per thread
  if (live && tid < D) {
    float w = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) w += part[ul][0][g][tid];
    fu[ul][tid] = be * (vc - w);
  }
  __syncthreads();
  // S'' = S' + k u^T, written back; the threads' parts of q_h^T S'', G heads
  // per pass
  for (int p = 0; p < NPASS; ++p) {
    if (p > 0) {
      // the previous pass read fq before its last barrier
      if (live) load_q(p);
      __syncthreads();
    }
    if (live) {
      float acc[G][4];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[h][i] = 0.f;
      if (p == 0) {
        float u4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u4[i] = fu[ul][4 * c4 + i];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          const float f = fk[ul][rg + RG * r];
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[r][i] = fmaf(f, u4[i], sv[r][i]);
        }
      }
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int dk = rg + RG * r;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float g = fq[ul][h][dk];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[h][i] = fmaf(g, sv[r][i], acc[h][i]);
        }
      }
      if (p == 0) {
        float* So = a.s_out + (int64_t)u * SE;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          f32x4_t* ptr = (f32x4_t*)(So + (rg + RG * r) * D + 4 * c4);
          if constexpr (NTMP)
            __builtin_nontemporal_store(sv[r], ptr);
          else
            *ptr = sv[r];
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[ul][h][rg][4 * c4 + i] = acc[h][i];
    }
    __syncthreads();
    if (live) {
      DT* op = (DT*)a.out + br * QW + (int64_t)j * GT * D + (int64_t)p * G * D;
      for (int i = tid; i < G * D; i += TPU) {
        const int h = i / D, d = i % D;
        float y = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g) y += part[ul][h][g][d];
        y *= a.scale;
        if constexpr (std::is_same_v<DT, uint16_t>)
          op[i] = (uint16_t)f32_to_bf16_bits(y);
        else
          op[i] = (DT)y;
      }
    }
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

// Launch shape of the decode kernel per head size: threads per unit and units
// per workgroup.  At head size 128 one 1024-thread workgroup per unit (4 state
// rows per thread) measured 182 us per step of the 8192-unit streaming
// workload, against 192 us for two 256-thread units per workgroup, 188 us for
// 512 x 2 and 183 us for 128 x 2 (a sweep of the shapes over this kernel).
template <int D>
struct DecodeShape {
  static constexpr int TPU = D == 128 ? 1024 : kThreads;
  static constexpr int UPB = D == 128 ? 1 : kDecodeUnits;
};

// (the shape follows the larger head size)
template <typename DT, int DK, int DV, int FM, bool NORM>
static void launch_k(bool ntmp, const DecodeArgs& a, int grid, hipStream_t st) {
  constexpr int DM = DK > DV ? DK : DV;
  constexpr int TPU = DecodeShape<DM>::TPU, UPB = DecodeShape<DM>::UPB;
  if (ntmp)
    hipLaunchKernelGGL((decode_kernel<DT, DK, DV, FM, NORM, true, TPU, UPB>), dim3(grid), dim3(TPU * UPB), 0, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<DT, DK, DV, FM, NORM, false, TPU, UPB>), dim3(grid), dim3(TPU * UPB), 0, st, a);
}

template <typename DT, int DK, int DV>
static hipError_t launch_d(int fm, int norm, const DecodeArgs& a, int units, hipStream_t st) {
  // states larger than the on-chip caches stream past them (non-temporal)
  const bool ntmp = (int64_t)units * DK * DV * 4 >= ((int64_t)256 << 20);
  constexpr int DM = DK > DV ? DK : DV;
  const int grid = (units + DecodeShape<DM>::UPB - 1) / DecodeShape<DM>::UPB;
  if (fm == kEluPlusOne) {
    if (norm) launch_k<DT, DK, DV, kEluPlusOne, true>(ntmp, a, grid, st);
    else launch_k<DT, DK, DV, kEluPlusOne, false>(ntmp, a, grid, st);
  } else {
    if (norm) launch_k<DT, DK, DV, kReluEps, true>(ntmp, a, grid, st);
    else launch_k<DT, DK, DV, kReluEps, false>(ntmp, a, grid, st);
  }
  return hipGetLastError();
}

template <typename DT, int DK>
static hipError_t launch_dv(int Dv, int fm, int norm, const DecodeArgs& a, int units, hipStream_t st) {
  switch (Dv) {
    case 32: return launch_d<DT, DK, 32>(fm, norm, a, units, st);
    case 64: return launch_d<DT, DK, 64>(fm, norm, a, units, st);
    default: return launch_d<DT, DK, 128>(fm, norm, a, units, st);
  }
}

template <typename DT>
static hipError_t launch_dt(int Dk, int Dv, int fm, int norm, const DecodeArgs& a, int units, hipStream_t st) {
  switch (Dk) {
    case 32: return launch_dv<DT, 32>(Dv, fm, norm, a, units, st);
    case 64: return launch_dv<DT, 64>(Dv, fm, norm, a, units, st);
    default: return launch_dv<DT, 128>(Dv, fm, norm, a, units, st);
  }
}

hipError_t launch_decode(int io, int Dk, int Dv, int fm, int norm, const DecodeArgs& a, int units,
                         hipStream_t st) {
  if (units <= 0) return hipSuccess;
  switch (io) {
    case kIoBF16: return launch_dt<uint16_t>(Dk, Dv, fm, norm, a, units, st);
    case kIoF16: return launch_dt<f16_t>(Dk, Dv, fm, norm, a, units, st);
    default: return launch_dt<float>(Dk, Dv, fm, norm, a, units, st);
  }
}

// Launch shape of the gated and delta steps: at head size 128 with up to 4
// query heads per pass one 1024-thread workgroup per unit (4 state rows per
// thread; the readout partials of 32 row groups take 16 KB of LDS per head),
// else two 256-thread units per workgroup.
template <int D, int G>
struct StepShape {
  static constexpr bool WIDE = D == 128 && G <= 4;
  static constexpr int TPU = WIDE ? 1024 : kThreads;
  static constexpr int UPB = WIDE ? 1 : kDecodeUnits;
};

// Query heads per readout pass for a kv head with G of them: the largest of
// 8, 4, 2, 1 that divides G.
static int head_tile(int G) { return G % 8 == 0 ? 8 : (G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1)); }

template <typename DT, int D, int G, bool PD, bool MP>
static void launch_gsp(const GatedStepArgs& a, hipStream_t st) {
  constexpr int TPU = StepShape<D, G>::TPU, UPB = StepShape<D, G>::UPB;
  const bool ntmp = (int64_t)a.units * D * D * 4 >= ((int64_t)256 << 20);
  const int grid = (a.units + UPB - 1) / UPB;
  if (ntmp)
    hipLaunchKernelGGL((gated_step_kernel<DT, D, G, true, PD, MP, TPU, UPB>), dim3(grid), dim3(TPU * UPB), 0, st, a);
  else
    hipLaunchKernelGGL((gated_step_kernel<DT, D, G, false, PD, MP, TPU, UPB>), dim3(grid), dim3(TPU * UPB), 0, st, a);
}

template <typename DT, int D, int G, bool MP>
static void launch_gs(const GatedStepArgs& a, hipStream_t st) {
  if (a.per_dim && a.decay)
    launch_gsp<DT, D, G, true, MP>(a, st);
  else
    launch_gsp<DT, D, G, false, MP>(a, st);
}

template <typename DT, int D>
static void launch_gs_g(int G, const GatedStepArgs& a0, hipStream_t st) {
  GatedStepArgs a = a0;
  a.heads = G;
  const int gp = head_tile(G);
  const bool mp = gp != G;
  switch (gp) {
    case 1: mp ? launch_gs<DT, D, 1, true>(a, st) : launch_gs<DT, D, 1, false>(a, st); break;
    case 2: mp ? launch_gs<DT, D, 2, true>(a, st) : launch_gs<DT, D, 2, false>(a, st); break;
    case 4: mp ? launch_gs<DT, D, 4, true>(a, st) : launch_gs<DT, D, 4, false>(a, st); break;
    default: mp ? launch_gs<DT, D, 8, true>(a, st) : launch_gs<DT, D, 8, false>(a, st); break;
  }
}

template <typename DT>
static void launch_gs_d(int D, int G, const GatedStepArgs& a, hipStream_t st) {
  switch (D) {
    case 32: launch_gs_g<DT, 32>(G, a, st); break;
    case 64: launch_gs_g<DT, 64>(G, a, st); break;
    default: launch_gs_g<DT, 128>(G, a, st); break;
  }
}

hipError_t launch_gated_step(int io, int D, int G, const GatedStepArgs& a, hipStream_t st) {
  if (a.units <= 0) return hipSuccess;
  switch (io) {
    case kIoBF16: launch_gs_d<uint16_t>(D, G, a, st); break;
    case kIoF16: launch_gs_d<f16_t>(D, G, a, st); break;
    default: launch_gs_d<float>(D, G, a, st); break;
  }
  return hipGetLastError();
}

template <typename DT, int D, int G, int DK, bool MP>
static void launch_dsp(const GatedStepArgs& a, hipStream_t st) {
  constexpr int TPU = StepShape<D, G>::TPU, UPB = StepShape<D, G>::UPB;
  const bool ntmp = (int64_t)a.units * D * D * 4 >= ((int64_t)256 << 20);
  const int grid = (a.units + UPB - 1) / UPB;
  if (ntmp)
    hipLaunchKernelGGL((delta_step_kernel<DT, D, G, true, DK, MP, TPU, UPB>), dim3(grid), dim3(TPU * UPB), 0, st, a);
  else
    hipLaunchKernelGGL((delta_step_kernel<DT, D, G, false, DK, MP, TPU, UPB>), dim3(grid), dim3(TPU * UPB), 0, st, a);
}

template <typename DT, int D, int G, bool MP>
static void launch_ds(const GatedStepArgs& a, hipStream_t st) {
  if (!a.decay)
    launch_dsp<DT, D, G, 0, MP>(a, st);
  else if (a.per_dim)
    launch_dsp<DT, D, G, 2, MP>(a, st);
  else
    launch_dsp<DT, D, G, 1, MP>(a, st);
}

template <typename DT, int D>
static void launch_ds_g(int G, const GatedStepArgs& a0, hipStream_t st) {
  GatedStepArgs a = a0;
  a.heads = G;
  const int gp = head_tile(G);
  const bool mp = gp != G;
  switch (gp) {
    case 1: mp ? launch_ds<DT, D, 1, true>(a, st) : launch_ds<DT, D, 1, false>(a, st); break;
    case 2: mp ? launch_ds<DT, D, 2, true>(a, st) : launch_ds<DT, D, 2, false>(a, st); break;
    case 4: mp ? launch_ds<DT, D, 4, true>(a, st) : launch_ds<DT, D, 4, false>(a, st); break;
    default: mp ? launch_ds<DT, D, 8, true>(a, st) : launch_ds<DT, D, 8, false>(a, st); break;
  }
}

template <typename DT>
static void launch_ds_d(int D, int G, const GatedStepArgs& a, hipStream_t st) {
  switch (D) {
    case 32: launch_ds_g<DT, 32>(G, a, st); break;
    case 64: launch_ds_g<DT, 64>(G, a, st); break;
    default: launch_ds_g<DT, 128>(G, a, st); break;
  }
}

hipError_t launch_delta_step(int io, int D, int G, const GatedStepArgs& a, hipStream_t st) {
  if (a.units <= 0) return hipSuccess;
  switch (io) {
    case kIoBF16: launch_ds_d<uint16_t>(D, G, a, st); break;
    case kIoF16: launch_ds_d<f16_t>(D, G, a, st); break;
    default: launch_ds_d<float>(D, G, a, st); break;
  }
  return hipGetLastError();
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
