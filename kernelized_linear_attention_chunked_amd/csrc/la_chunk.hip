// Chunk-parallel kernels for causal and non-causal kernelized linear attention.
//
// One templated kernel, three modes:
//   kCausal : causal prefill ("[Feature] LinearAttention layer for Keras",
//             sections "Mathematical definition / Causal", "Masking / Causal",
//             "Streaming State").  Per chunk of 64 tokens it forms
//               A^T = phiK phiQ^T (lower triangle, diagonal included),
//               N^T = V^T A^T + S_prev^T phiQ^T,
//             divides by the normaliser and stores the outputs, then adds
//             phiK^T V to the running state S (carried in registers).
//   kState  : only the state increment  sum_t phiK_t^T V_t  over a segment of
//             chunks (the partial sums of a split sequence, and the non-causal
//             reduction of "Mathematical definition / Non-causal").
//   kApply  : only  y = phiQ S / (phiQ Z + eps)  with a fixed S (the non-causal
//             readout).
// The operator page ("LinearAttention", ai.onnx v27, "Description") allows any
// chunk-parallel evaluation with the sequential result; chunking changes only
// the summation order.
//
// The normaliser rides along in the same MFMAs: V^T gets 16 extra rows of
// ones and S gets 16 extra columns holding Z, so the extra output tile of
// N^T holds  sum_j A_ij + phiQ_i . Z_prev  (the denominator before eps), and
// the extra state tile accumulates Z exactly like S.
//
// Work split inside a 256-thread workgroup (one (batch, head) unit and one
// segment of chunks):
//   wave w owns query rows [16w, 16w+16) of the chunk (A^T tiles jt <= w,
//   N^T, outputs) and a contiguous quarter of the 16x16 tiles of S.
// LDS holds phiK in natural [token][dk] layout, V transposed [dv][token] and a
// copy of S transposed [dv][dk] in the operand dtype.  The next chunk's q/k/v
// are loaded into registers while the current chunk is being computed.
#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

enum ChunkMode { kCausal = 0, kState = 1, kApply = 2 };

template <typename DT, int D, int FM, bool NORM, int MODE>
__global__ __launch_bounds__(kThreads, 2) void chunk_kernel(ChunkArgs a) {
  using O = Op<DT>;
  constexpr int VEC = O::VEC, KB = O::KB, ESZ = O::ESZ;
  constexpr int NDT = D / 16;                      // 16-wide tiles along dk or dv
  constexpr int NVT = NDT + (NORM ? 1 : 0);        // dv tiles plus the normaliser tile
  constexpr int CB = D / VEC;                      // 16-byte blocks per row
  constexpr int NTOK = kChunk * CB / kThreads;     // tokens per thread in k/v loads
  constexpr int NQ = D / KB;                       // operand vectors per q row per lane
  constexpr int NKS = kChunk / KB;                 // vector-steps over the chunk's tokens
  constexpr int PADE = 16 / ESZ;                   // 16 bytes of padding per LDS row
  constexpr int KN_LD = D + PADE;
  constexpr int VT_LD = kChunk + PADE;
  constexpr int SB_LD = D + PADE;
  constexpr bool USE_KV = MODE != kApply;
  constexpr bool USE_Q = MODE != kState;
  constexpr bool USE_SB = MODE != kState;
  constexpr int KN_BYTES = USE_KV ? kChunk * KN_LD * ESZ : 0;
  constexpr int VT_BYTES = USE_KV ? NVT * 16 * VT_LD * ESZ : 0;
  constexpr int SB_BYTES = USE_SB ? NVT * 16 * SB_LD * ESZ : 0;
  constexpr int NS = NDT * NVT;                    // 16x16 tiles of the (extended) state
  constexpr int TPW = (NS + 3) / 4;                // state tiles per wave
  static_assert(NTOK >= 1 && NQ >= 1, "unsupported head size");

  __shared__ __align__(16) unsigned char smem[KN_BYTES + VT_BYTES + SB_BYTES + 16];
  DT* Kn = (DT*)smem;
  DT* Vt = (DT*)(smem + KN_BYTES);
  DT* Sb = (DT*)(smem + KN_BYTES + VT_BYTES);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lr = l & 15, lg = l >> 4;
  const int bid = blockIdx.x;
  const int u = bid / a.seg_count;
  const int s = a.seg_first + bid % a.seg_count;
  const int H = a.H, T = a.T;
  const int b = u / H, h = u % H;
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int c0 = s * a.seg_chunks;
  const int c1 = min(c0 + a.seg_chunks, nchunks);
  const int HD = H * D;
  const int64_t unit_off = (int64_t)b * T * HD + (int64_t)h * D;
  const DT* qb = (const DT*)a.q + unit_off;
  const DT* kb = (const DT*)a.k + unit_off;
  const DT* vb = (const DT*)a.v + unit_off;
  DT* ob = (DT*)a.out + unit_off;
  const uint8_t* mb = a.mask ? a.mask + (int64_t)b * T : nullptr;
  const float eps = a.eps;

  // ---- running state: wave w owns tiles tau = w*TPW + i of the (NDT x NVT) grid
  f32x4_t sacc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) sacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (MODE != kState) {
    const float* sin = a.s_in ? a.s_in + u * a.s_in_u + s * a.s_in_s : nullptr;
    const float* zin = a.z_in ? a.z_in + u * a.z_in_u + s * a.z_in_s : nullptr;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tau = w * TPW + i;
      if (tau < NS) {
        const int rt = tau / NVT, ct = tau % NVT;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int dk = 16 * rt + 4 * lg + q;
          float val = 0.f;
          if (ct < NDT) {
            if (sin) val = sin[dk * D + 16 * ct + lr];
          } else {
            if (zin) val = zin[dk];
          }
          sacc[i][q] = val;
        }
      }
    }
  }

  // S (and Z in the extra rows) -> LDS, transposed [dv][dk], operand dtype.
  auto write_sb = [&]() {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tau = w * TPW + i;
      if (tau < NS) {
        const int rt = tau / NVT, ct = tau % NVT;
        DT* p = Sb + (16 * ct + lr) * SB_LD + 16 * rt + 4 * lg;
        if constexpr (ESZ == 2) {
          u32x2_t v2;
          v2[0] = pack_bf16x2(sacc[i][0], sacc[i][1]);
          v2[1] = pack_bf16x2(sacc[i][2], sacc[i][3]);
          *(u32x2_t*)p = v2;
        } else {
          *(f32x4_t*)p = sacc[i];
        }
      }
    }
  };
  if constexpr (USE_SB) write_sb();
  if constexpr (USE_KV && NORM) {
    // rows D..D+15 of V^T are ones: they turn A V into the row sums of A
    for (int idx = tid; idx < 16 * kChunk; idx += kThreads) {
      const int r = D + idx / kChunk, c = idx % kChunk;
      if constexpr (ESZ == 2)
        ((uint16_t*)Vt)[r * VT_LD + c] = 0x3f80;  // bf16 1.0
      else
        ((float*)Vt)[r * VT_LD + c] = 1.f;
    }
  }

  // ---- prefetch registers
  const int cb = tid % CB, tg = tid / CB;
  u32x4_t pk[USE_KV ? NTOK : 1], pv[USE_KV ? NTOK : 1], pq[USE_Q ? NQ : 1];
  uint32_t kvalid = 0, qvalid = 0;
  auto prefetch = [&](int c) {
    const int tb = c * kChunk;
    if constexpr (USE_KV) {
      kvalid = 0;
#pragma unroll
      for (int n = 0; n < NTOK; ++n) {
        const int tok = tb + tg * NTOK + n;
        if (tok < T) {
          const int64_t off = (int64_t)tok * HD + cb * VEC;
          pk[n] = ld16(kb + off);
          pv[n] = ld16(vb + off);
          const uint32_t ok = mb ? (mb[tok] != 0) : 1u;
          kvalid |= ok << n;
        } else {
          pk[n] = u32x4_t{0u, 0u, 0u, 0u};
          pv[n] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
    if constexpr (USE_Q) {
      const int tok = tb + 16 * w + lr;
      qvalid = 0;
      if (tok < T) {
        const int64_t off = (int64_t)tok * HD + VEC * lg;
#pragma unroll
        for (int m = 0; m < NQ; ++m) pq[m] = ld16(qb + off + KB * m);
        qvalid = mb ? (mb[tok] != 0) : 1u;
      } else {
#pragma unroll
        for (int m = 0; m < NQ; ++m) pq[m] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };

  // ---- stage: prefetched registers -> phi(K) [token][dk] and V^T [dv][token] in
  // LDS, phi(Q) operand registers.  Invalid tokens are selected to zero (a
  // masked token must not reach the state, whatever its values).
  u32x4_t qop[USE_Q ? NQ : 1];
  bool qok = false;  // validity of this lane's query row in the chunk being computed
  auto stage = [&]() {
    if constexpr (USE_KV) {
#pragma unroll
      for (int n = 0; n < NTOK; ++n) {
        const bool ok = (kvalid >> n) & 1u;
        float f[VEC];
        O::unpack(pk[n], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) f[e] = ok ? phi<FM>(f[e], eps) : 0.f;
        st16(Kn + (tg * NTOK + n) * KN_LD + cb * VEC, O::pack(f));
        if (!ok) pv[n] = u32x4_t{0u, 0u, 0u, 0u};
      }
      // transposed V: element e of every loaded vector goes to row cb*VEC+e,
      // the NTOK consecutive tokens of this thread side by side.
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        DT* p = Vt + (cb * VEC + e) * VT_LD + tg * NTOK;
        if constexpr (ESZ == 2) {
          uint32_t hw[NTOK];
#pragma unroll
          for (int n = 0; n < NTOK; ++n) hw[n] = (pv[n][e >> 1] >> (16 * (e & 1))) & 0xffffu;
          if constexpr (NTOK == 1) {
            *(uint16_t*)p = (uint16_t)hw[0];
          } else if constexpr (NTOK == 2) {
            *(uint32_t*)p = hw[0] | (hw[1] << 16);
          } else {
#pragma unroll
            for (int n = 0; n < NTOK; n += 4) {
              u32x2_t v2;
              v2[0] = hw[n] | (hw[n + 1] << 16);
              v2[1] = hw[n + 2] | (hw[n + 3] << 16);
              *(u32x2_t*)(p + n) = v2;
            }
          }
        } else {
          float fv[NTOK];
#pragma unroll
          for (int n = 0; n < NTOK; ++n) fv[n] = __uint_as_float(pv[n][e]);
          if constexpr (NTOK == 1) {
            *(float*)p = fv[0];
          } else if constexpr (NTOK == 2) {
            *(float2*)p = make_float2(fv[0], fv[1]);
          } else {
#pragma unroll
            for (int n = 0; n < NTOK; n += 4)
              *(f32x4_t*)(p + n) = f32x4_t{fv[n], fv[n + 1], fv[n + 2], fv[n + 3]};
          }
        }
      }
    }
    if constexpr (USE_Q) {
      const bool ok = qvalid != 0;
      qok = ok;
#pragma unroll
      for (int m = 0; m < NQ; ++m) {
        float f[VEC];
        O::unpack(pq[m], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) f[e] = ok ? phi<FM>(f[e], eps) : 0.f;
        qop[m] = O::pack(f);
      }
    }
  };

  // ---- per-chunk compute
  auto compute = [&](int c) {
    if constexpr (USE_Q) {
      f32x4_t nacc[NVT];
#pragma unroll
      for (int ct = 0; ct < NVT; ++ct) nacc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (MODE == kCausal) {
        // A^T tile jt: rows = keys 16jt + 4lg + q, column = own query 16w + lr.
        // A operand: phiK rows from LDS; B operand: phiQ registers (contraction over dk).
        f32x4_t at[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          at[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (jt <= w) {
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
              const u32x4_t av = ld16(Kn + (16 * jt + lr) * KN_LD + KB * m + VEC * lg);
              O::mma(at[jt], av, qop[m]);
            }
            if (jt == w) {  // causal mask inside the diagonal tile: key <= query
#pragma unroll
              for (int q = 0; q < 4; ++q) at[jt][q] = (4 * lg + q <= lr) ? at[jt][q] : 0.f;
            }
          }
        }
        // N^T += V^T A^T: contraction over keys.  The B operand is A^T straight
        // from the accumulators: lane group lg holds keys 16jt + 4lg + q, so the
        // A operand (V^T rows) reads the same keys.
        if constexpr (ESZ == 2) {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            if (2 * p <= w) {
              const int j0 = 32 * p + 4 * lg, j1 = j0 + 16;
              // phi >= 0 makes every A entry positive with a large common
              // part, so one bf16 rounding of A would dominate the error;
              // A = hi + lo, both bf16, keeps it to ~2^-16 relative.
              u32x4_t bh, bl;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const f32x4_t& src = at[2 * p + (e >> 1)];
                const float x0 = src[2 * (e & 1)], x1 = src[2 * (e & 1) + 1];
                const uint32_t h0 = f32_to_bf16_bits(x0), h1 = f32_to_bf16_bits(x1);
                bh[e] = h0 | (h1 << 16);
                bl[e] = pack_bf16x2(x0 - bf16_bits_to_f32(h0), x1 - bf16_bits_to_f32(h1));
              }
#pragma unroll
              for (int ct = 0; ct < NVT; ++ct) {
                const DT* vr = Vt + (16 * ct + lr) * VT_LD;
                const u32x2_t lo = *(const u32x2_t*)(vr + j0);
                const u32x2_t hi = *(const u32x2_t*)(vr + j1);
                const u32x4_t av = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
                O::mma(nacc[ct], av, bh);
                O::mma(nacc[ct], av, bl);
              }
            }
          }
        } else {
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) {
            if (jt <= w) {
#pragma unroll
              for (int ct = 0; ct < NVT; ++ct) {
                const f32x4_t av = *(const f32x4_t*)(Vt + (16 * ct + lr) * VT_LD + 16 * jt + 4 * lg);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                  nacc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], at[jt][q], nacc[ct], 0, 0, 0);
              }
            }
          }
        }
      }
      // N^T += S^T phiQ^T (state before this chunk): contraction over dk.
#pragma unroll
      for (int ct = 0; ct < NVT; ++ct) {
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
          const u32x4_t av = ld16(Sb + (16 * ct + lr) * SB_LD + KB * m + VEC * lg);
          O::mma(nacc[ct], av, qop[m]);
        }
      }
      // epilogue: lane holds query 16w + lr, value dims 16ct + 4lg + (0..3)
      const int tok = c * kChunk + 16 * w + lr;
      if (tok < T) {
        const bool ok = qok;
        float rden = 1.f;
        if constexpr (NORM) rden = 1.f / (nacc[NDT][0] + eps);
        DT* orow = ob + (int64_t)tok * HD + 4 * lg;
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) {
          float y0 = nacc[ct][0] * rden, y1 = nacc[ct][1] * rden;
          float y2 = nacc[ct][2] * rden, y3 = nacc[ct][3] * rden;
          if (!ok) y0 = y1 = y2 = y3 = 0.f;
          store4(orow + 16 * ct, y0, y1, y2, y3);
        }
      }
    }
    if constexpr (USE_KV) {
      // S += phiK^T V over the chunk's tokens.  A operand: phiK^T rows (dk) read
      // column-wise from the natural layout; B operand: V^T rows (dv).  Lane
      // group lg carries tokens KB*m + VEC*lg + e.
      u32x4_t kop[NKS];
      int cur_rt = -1;
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int tau = w * TPW + i;
        if (tau < NS) {
          const int rt = tau / NVT, ct = tau % NVT;
          if (rt != cur_rt) {
            cur_rt = rt;
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
              const DT* kc = Kn + (KB * m + VEC * lg) * KN_LD + 16 * rt + lr;
              if constexpr (ESZ == 2) {
                const uint16_t* k16 = (const uint16_t*)kc;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  kop[m][e] = (uint32_t)k16[(2 * e) * KN_LD] | ((uint32_t)k16[(2 * e + 1) * KN_LD] << 16);
              } else {
                const float* k32 = (const float*)kc;
#pragma unroll
                for (int e = 0; e < 4; ++e) kop[m][e] = __float_as_uint(k32[e * KN_LD]);
              }
            }
          }
#pragma unroll
          for (int m = 0; m < NKS; ++m) {
            const u32x4_t bv = ld16(Vt + (16 * ct + lr) * VT_LD + KB * m + VEC * lg);
            O::mma(sacc[i], kop[m], bv);
          }
        }
      }
    }
  };

  if (c0 < c1) prefetch(c0);
  for (int c = c0; c < c1; ++c) {
    stage();
    __syncthreads();
    if (c + 1 < c1) prefetch(c + 1);
    compute(c);
    if constexpr (MODE != kApply) {
      __syncthreads();
      if constexpr (MODE == kCausal) write_sb();
    }
  }

  // ---- state out
  float* sout = nullptr;
  float* zout = nullptr;
  if constexpr (MODE == kCausal) {
    if (s == a.nseg_total - 1) {
      sout = a.s_out ? a.s_out + u * a.s_out_u : nullptr;
      zout = a.z_out ? a.z_out + u * a.z_out_u : nullptr;
    }
  } else if constexpr (MODE == kState) {
    sout = a.s_out + u * a.s_out_u + (s + a.out_slot_off) * a.s_out_s;
    zout = a.z_out ? a.z_out + u * a.z_out_u + (s + a.out_slot_off) * a.z_out_s : nullptr;
  }
  if constexpr (MODE != kApply) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tau = w * TPW + i;
      if (tau < NS) {
        const int rt = tau / NVT, ct = tau % NVT;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int dk = 16 * rt + 4 * lg + q;
          if (ct < NDT) {
            if (sout) sout[dk * D + 16 * ct + lr] = sacc[i][q];
          } else {
            if (zout && lr == 0) zout[dk] = sacc[i][q];
          }
        }
      }
    }
  }
}

// Exclusive prefix over segment partial states, in place.  Slot s of unit u
// holds the increment of segment s-1 on entry (slot 0 is ignored) and the
// state before segment s on exit; slot 0 receives the caller's initial state
// (or zeros).  One thread per state element, sequential over segments.
__global__ __launch_bounds__(kThreads) void seg_prefix_kernel(float* ws_s, float* ws_z,
                                                              const float* s_in, const float* z_in,
                                                              int U, int nseg, int D, int norm) {
  const int64_t per = (int64_t)D * D + (norm ? D : 0);
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)U * per) return;
  const int u = (int)(idx / per);
  const int e = (int)(idx % per);
  float* base;
  int64_t stride;
  float acc;
  if (e < D * D) {
    base = ws_s + (int64_t)u * nseg * D * D + e;
    stride = (int64_t)D * D;
    acc = s_in ? s_in[(int64_t)u * D * D + e] : 0.f;
  } else {
    const int ez = e - D * D;
    base = ws_z + (int64_t)u * nseg * D + ez;
    stride = D;
    acc = z_in ? z_in[(int64_t)u * D + ez] : 0.f;
  }
  base[0] = acc;
  for (int s = 1; s < nseg; ++s) {
    acc += base[s * stride];
    base[s * stride] = acc;
  }
}

// Sum of all segment partials of a unit, in fixed segment order, into slot 0.
__global__ __launch_bounds__(kThreads) void seg_sum_kernel(float* ws_s, float* ws_z, int U,
                                                           int nseg, int D, int norm) {
  const int64_t per = (int64_t)D * D + (norm ? D : 0);
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)U * per) return;
  const int u = (int)(idx / per);
  const int e = (int)(idx % per);
  float* base;
  int64_t stride;
  if (e < D * D) {
    base = ws_s + (int64_t)u * nseg * D * D + e;
    stride = (int64_t)D * D;
  } else {
    base = ws_z + (int64_t)u * nseg * D + (e - D * D);
    stride = D;
  }
  float acc = 0.f;
  for (int s = 0; s < nseg; ++s) acc += base[s * stride];
  base[0] = acc;
}

// ---------------------------------------------------------------------------
// host-side launchers

template <typename DT, int D, int FM, bool NORM, int MODE>
static hipError_t launch_one(const ChunkArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((chunk_kernel<DT, D, FM, NORM, MODE>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <typename DT, int D, int FM, bool NORM>
static hipError_t launch_mode(int mode, const ChunkArgs& a, int grid, hipStream_t st) {
  switch (mode) {
    case kCausal: return launch_one<DT, D, FM, NORM, kCausal>(a, grid, st);
    case kState: return launch_one<DT, D, FM, NORM, kState>(a, grid, st);
    default: return launch_one<DT, D, FM, NORM, kApply>(a, grid, st);
  }
}

template <typename DT, int D>
static hipError_t launch_d(int mode, int fm, int norm, const ChunkArgs& a, int grid, hipStream_t st) {
  if (fm == kEluPlusOne)
    return norm ? launch_mode<DT, D, kEluPlusOne, true>(mode, a, grid, st)
                : launch_mode<DT, D, kEluPlusOne, false>(mode, a, grid, st);
  return norm ? launch_mode<DT, D, kReluEps, true>(mode, a, grid, st)
              : launch_mode<DT, D, kReluEps, false>(mode, a, grid, st);
}

template <typename DT>
static hipError_t launch_dt(int mode, int D, int fm, int norm, const ChunkArgs& a, int grid,
                            hipStream_t st) {
  switch (D) {
    case 32: return launch_d<DT, 32>(mode, fm, norm, a, grid, st);
    case 64: return launch_d<DT, 64>(mode, fm, norm, a, grid, st);
    default: return launch_d<DT, 128>(mode, fm, norm, a, grid, st);
  }
}

hipError_t launch_chunk(int mode, int bf16, int D, int fm, int norm, const ChunkArgs& a, int grid,
                        hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  return bf16 ? launch_dt<uint16_t>(mode, D, fm, norm, a, grid, st)
              : launch_dt<float>(mode, D, fm, norm, a, grid, st);
}

hipError_t launch_seg_prefix(float* ws_s, float* ws_z, const float* s_in, const float* z_in, int U,
                             int nseg, int D, int norm, hipStream_t st) {
  const int64_t n = (int64_t)U * ((int64_t)D * D + (norm ? D : 0));
  const int grid = (int)((n + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(seg_prefix_kernel, dim3(grid), dim3(kThreads), 0, st, ws_s, ws_z, s_in, z_in,
                     U, nseg, D, norm);
  return hipGetLastError();
}

hipError_t launch_seg_sum(float* ws_s, float* ws_z, int U, int nseg, int D, int norm,
                          hipStream_t st) {
  const int64_t n = (int64_t)U * ((int64_t)D * D + (norm ? D : 0));
  const int grid = (int)((n + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(seg_sum_kernel, dim3(grid), dim3(kThreads), 0, st, ws_s, ws_z, U, nseg, D, norm);
  return hipGetLastError();
}

}  // namespace la
