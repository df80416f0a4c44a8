// Whole-sequence token-by-token evaluation of the gated and delta recurrences
// (the LinearAttention operator page, ai.onnx since version 27, "Description":
// the recurrence is defined one token at a time),
//   S_t = E_t S_{t-1} + k_t u_t^T,  u_t = v_t ("gated") or
//   u_t = beta_t (v_t - (E_t S_{t-1})^T k_t) ("gated_delta"),
//   o_t = scale q_t^T S_t per query head,
// with the state in registers from the first token to the last.  It serves
// fp32 inputs at head size 128 with a per-key-dim decay, whose fp32 chunk tiles
// and table of cumulative decays do not fit the LDS of the chunk kernels.
//
// The columns of S evolve independently under both rules: E_t scales rows, the
// rank-1 term adds k_t u_t^T, and the delta correction (E_t S)^T k_t is taken
// column by column.  So a workgroup holds 32 columns of one unit's state and
// writes those 32 columns of every output: (unit, query-head group, column
// group) workgroups, four per head of 128 values.  Thread (row group rq, column
// c) keeps rows [16 rq, 16 rq + 16) of column c.
//
// Inputs come in blocks of W tokens plus the next block's first token, loaded
// into registers while the previous block is evaluated and then parked in LDS
// (k, exp(g), the group's queries, the workgroup's v columns and beta per
// token).  Each token takes one barrier: its readout partials over the row
// groups (and, for the delta rule, the next token's (E S)^T k partials) go to
// one of two alternating LDS buffers and are summed after it.
#include "la_launch.hpp"
#include "la_device.hpp"

namespace la {

constexpr int kRecurThreads = 256;
constexpr int kRecurCols = 32;                                // state columns per workgroup
constexpr int kRecurRowGroups = kRecurThreads / kRecurCols;  // 8

// Floats of one token slot (offsets of k, exp(g), the queries, v and beta,
// each 16-byte aligned), tokens per block, partial-sum rows, LDS bytes.
template <int D, int GW, int DK, bool DELTA>
struct RecurTok {
  static constexpr int NEV = DK == 2 ? D : (DK == 1 ? 1 : 0);
  static constexpr int OK = 0, OE = D, OQ = ((D + NEV + 3) / 4) * 4;
  static constexpr int OV = OQ + GW * D, OB = OV + kRecurCols;
  static constexpr int F = ((OB + (DELTA ? 1 : 0) + 3) / 4) * 4;
  static constexpr int W0 = 16384 / F - 1;  // block and lookahead slot within 64 KB
  static constexpr int W = W0 > 16 ? 16 : (W0 < 1 ? 1 : W0);
  static constexpr int NRED = GW + (DELTA ? 1 : 0);
  static constexpr int FLOATS = (W + 1) * F + 2 * NRED * kRecurThreads;
};

template <typename IT, int D, int GW, int DK, bool DELTA>
__global__ __launch_bounds__(kRecurThreads) void recur_kernel(RecurArgs a) {
  using TS = RecurTok<D, GW, DK, DELTA>;
  constexpr int NTH = kRecurThreads, DC = kRecurCols, NRG = kRecurRowGroups, RPT = D / NRG;
  constexpr int NCG = D / DC;
  constexpr int W = TS::W, F = TS::F, NRED = TS::NRED;
  constexpr int OK = TS::OK, OE = TS::OE, OQ = TS::OQ, OV = TS::OV, OB = TS::OB;
  static_assert(RPT % 4 == 0 && D % DC == 0 && F % 4 == 0 && OQ % 4 == 0, "unsupported shape");
  __shared__ __align__(16) float lds[TS::FLOATS];
  float* blk = lds;                // [W + 1][F] token slots
  float* red = lds + (W + 1) * F;  // [2][NRED][NRG][DC] partial sums

  const int tid = threadIdx.x;
  const int col = tid % DC, rq = tid / DC;
  // column group slowest, so that the column groups of a unit share an XCD
  // when the units and head groups come in multiples of 8
  const int per_cg = a.units * a.hg_count;
  const int cg = blockIdx.x / per_cg;
  const int rest = blockIdx.x % per_cg;
  const int u = rest / a.hg_count;
  const int hg = a.hg_first + rest % a.hg_count;
  const int hs = a.hsplit > 1 ? a.hsplit : 1;
  const int b = u / a.Hkv, j = u % a.Hkv;
  const int T = a.T;
  const int64_t QS = (int64_t)a.Hq * D, KS = (int64_t)a.Hkv * D;
  const IT* qb = (const IT*)a.q + (int64_t)b * T * QS + (int64_t)(j * GW * hs + hg * GW) * D;
  IT* ob = (IT*)a.out + (int64_t)b * T * QS + (int64_t)(j * GW * hs + hg * GW) * D + cg * DC;
  const IT* kb = (const IT*)a.k + (int64_t)b * T * KS + (int64_t)j * D;
  const IT* vb = (const IT*)a.v + (int64_t)b * T * KS + (int64_t)j * D + cg * DC;
  const IT* gb = DK == 2 ? (const IT*)a.decay + (int64_t)b * T * KS + (int64_t)j * D
                         : (DK == 1 ? (const IT*)a.decay + (int64_t)b * T * a.Hkv + j : nullptr);
  const int64_t GS = DK == 2 ? KS : a.Hkv;
  const int bh = a.beta_heads;
  const IT* bb = DELTA ? (const IT*)a.beta + (int64_t)b * T * bh + (bh > 1 ? j : 0) : nullptr;
  const float* sin = a.s_in ? a.s_in + (int64_t)u * D * D : nullptr;
  float* sout = (hg == 0 && a.s_out) ? a.s_out + (int64_t)u * D * D : nullptr;
  auto ld = [](const IT* p) { return Io<IT>::to_f32(sizeof(IT) == 4 ? *(const uint32_t*)p : (uint32_t)*(const uint16_t*)p); };

  // ---- block loads: element f = tid + NTH * i of each field, slot f / (field size)
  constexpr int NK = ((W + 1) * D + NTH - 1) / NTH;
  constexpr int NE = DK == 2 ? NK : 1;
  constexpr int NQ = ((W + 1) * GW * D + NTH - 1) / NTH;
  constexpr int NV = ((W + 1) * DC + NTH - 1) / NTH;
  float rk[NK], re[NE], rqv[NQ], rv[NV], rb = 0.f;
  // token of slot s of the block at tb, clamped into the sequence (slots past
  // the end are loaded from the last token and never read)
  auto tok = [&](int tb, int s) { return min(tb + s, T - 1); };
  auto fetch = [&](int tb) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int f = tid + NTH * i, s = min(f / D, W), d = f % D;
      rk[i] = ld(kb + (int64_t)tok(tb, s) * KS + d);
      if constexpr (DK == 2) re[i] = ld(gb + (int64_t)tok(tb, s) * GS + d);
    }
    if constexpr (DK == 1) re[0] = ld(gb + (int64_t)tok(tb, min(tid, W)) * GS);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int f = tid + NTH * i, s = min(f / (GW * D), W), o = f % (GW * D);
      rqv[i] = ld(qb + (int64_t)tok(tb, s) * QS + o);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int f = tid + NTH * i, s = min(f / DC, W), c = f % DC;
      rv[i] = ld(vb + (int64_t)tok(tb, s) * KS + c);
    }
    if constexpr (DELTA) rb = ld(bb + (int64_t)tok(tb, min(tid, W)) * bh);
  };
  auto park = [&]() {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int f = tid + NTH * i;
      if (f < (W + 1) * D) {
        blk[(f / D) * F + OK + f % D] = rk[i];
        if constexpr (DK == 2) blk[(f / D) * F + OE + f % D] = __expf(re[i]);
      }
    }
    if constexpr (DK == 1)
      if (tid <= W) blk[tid * F + OE] = __expf(re[0]);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int f = tid + NTH * i;
      if (f < (W + 1) * GW * D) blk[(f / (GW * D)) * F + OQ + f % (GW * D)] = rqv[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int f = tid + NTH * i;
      if (f < (W + 1) * DC) blk[(f / DC) * F + OV + f % DC] = rv[i];
    }
    if constexpr (DELTA)
      if (tid <= W) blk[tid * F + OB] = rb;
  };
  // RPT consecutive floats of a slot field at row RPT * rq
  auto rows = [&](const float* p, float (&x)[RPT]) {
#pragma unroll
    for (int r = 0; r < RPT; r += 4) {
      const f32x4_t y = *(const f32x4_t*)(p + RPT * rq + r);
      x[r] = y[0];
      x[r + 1] = y[1];
      x[r + 2] = y[2];
      x[r + 3] = y[3];
    }
  };

  float sv[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) sv[r] = sin ? sin[(int64_t)(RPT * rq + r) * D + cg * DC + col] : 0.f;

  // delta rule: partial sum over the thread's rows of (E S)^T k for the token
  // in slot `sl`, into row GW of partial buffer `buf`
  auto w_partial = [&](const float* sl, int buf) {
    float kk[RPT];
    rows(sl + OK, kk);
    float p = 0.f;
    if constexpr (DK == 2) {
      float ee[RPT];
      rows(sl + OE, ee);
#pragma unroll
      for (int r = 0; r < RPT; ++r) p = fmaf(ee[r] * kk[r], sv[r], p);
    } else {
#pragma unroll
      for (int r = 0; r < RPT; ++r) p = fmaf(kk[r], sv[r], p);
      if constexpr (DK == 1) p *= sl[OE];
    }
    red[((buf * NRED + GW) * NRG + rq) * DC + col] = p;
  };

  fetch(0);
  int n = 0;  // tokens done
  for (int tb = 0; tb < T; tb += W) {
    park();
    __syncthreads();
    if (tb + W < T) fetch(tb + W);
    if constexpr (DELTA) {
      if (tb == 0) {
        w_partial(blk, 1);
        __syncthreads();
      }
    }
    const int nt = min(W, T - tb);
    for (int i = 0; i < nt; ++i, ++n) {
      const int t = tb + i;
      const float* sl = blk + i * F;
      // S' = E S
      if constexpr (DK == 2) {
        float ee[RPT];
        rows(sl + OE, ee);
#pragma unroll
        for (int r = 0; r < RPT; ++r) sv[r] *= ee[r];
      } else if constexpr (DK == 1) {
        const float e = sl[OE];
#pragma unroll
        for (int r = 0; r < RPT; ++r) sv[r] *= e;
      }
      // u = v, or beta (v - (E S)^T k) from the partials summed after the last barrier
      float uc = sl[OV + col];
      if constexpr (DELTA) {
        const float* pw = red + ((((n + 1) & 1) * NRED + GW) * NRG) * DC + col;
        float w = 0.f;
#pragma unroll
        for (int g = 0; g < NRG; ++g) w += pw[g * DC];
        uc = sl[OB] * (uc - w);
      }
      // S'' = S' + k u^T
      {
        float kk[RPT];
        rows(sl + OK, kk);
#pragma unroll
        for (int r = 0; r < RPT; ++r) sv[r] = fmaf(kk[r], uc, sv[r]);
      }
      // readout partials of the GW heads
      float* rd = red + (n & 1) * NRED * NRG * DC;
#pragma unroll
      for (int h = 0; h < GW; ++h) {
        float qq[RPT];
        rows(sl + OQ + h * D, qq);
        float p = 0.f;
#pragma unroll
        for (int r = 0; r < RPT; ++r) p = fmaf(qq[r], sv[r], p);
        rd[(h * NRG + rq) * DC + col] = p;
      }
      if constexpr (DELTA)
        if (t + 1 < T) w_partial(sl + F, n & 1);
      __syncthreads();
      if (tid < GW * DC) {
        const int h = tid / DC, c = tid % DC;
        float y = 0.f;
#pragma unroll
        for (int g = 0; g < NRG; ++g) y += rd[(h * NRG + g) * DC + c];
        y *= a.scale;
        IT* op = ob + (int64_t)t * QS + (int64_t)h * D + c;
        if constexpr (std::is_same_v<IT, uint16_t>)
          *op = (uint16_t)f32_to_bf16_bits(y);
        else
          *op = (IT)y;
      }
    }
  }
  if (sout) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) sout[(int64_t)(RPT * rq + r) * D + cg * DC + col] = sv[r];
  }
}

template <typename IT, int D, int GW, int DK>
static void launch_rd(bool delta, const RecurArgs& a, hipStream_t st) {
  const int grid = a.units * a.hg_count * (D / kRecurCols);
  if (delta)
    hipLaunchKernelGGL((recur_kernel<IT, D, GW, DK, true>), dim3(grid), dim3(kRecurThreads), 0, st, a);
  else
    hipLaunchKernelGGL((recur_kernel<IT, D, GW, DK, false>), dim3(grid), dim3(kRecurThreads), 0, st, a);
}

template <typename IT, int D>
static void launch_rg(int G, int dk, bool delta, const RecurArgs& a, hipStream_t st) {
  auto go = [&](auto gw) {
    constexpr int GW = decltype(gw)::value;
    switch (dk) {
      case 0: launch_rd<IT, D, GW, 0>(delta, a, st); break;
      case 1: launch_rd<IT, D, GW, 1>(delta, a, st); break;
      default: launch_rd<IT, D, GW, 2>(delta, a, st); break;
    }
  };
  switch (G) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    default: go(std::integral_constant<int, 8>{}); break;
  }
}

hipError_t launch_recur(int io, int D, int G, int decay_kind, int delta, const RecurArgs& args, hipStream_t st) {
  if (args.units <= 0 || args.T <= 0) return hipSuccess;
  // head size 128 only: the smaller ones fit the chunk kernels
  if (D != 128) return hipErrorInvalidValue;
  auto run = [&](const RecurArgs& a) {
    switch (io) {
      case kIoBF16: launch_rg<uint16_t, 128>(G, decay_kind, delta != 0, a, st); break;
      case kIoF16: launch_rg<f16_t, 128>(G, decay_kind, delta != 0, a, st); break;
      default: launch_rg<float, 128>(G, decay_kind, delta != 0, a, st); break;
    }
  };
  RecurArgs a = args;
  const int hs = a.hsplit > 1 ? a.hsplit : 1;
  if (hs > 1 && a.s_in && a.s_in == a.s_out) {
    // the state updated in place with several query-head groups: the groups
    // that only read it run first, then group 0, which also writes it
    a.hg_first = 1;
    a.hg_count = hs - 1;
    run(a);
    a.hg_first = 0;
    a.hg_count = 1;
    run(a);
  } else {
    a.hg_first = 0;
    a.hg_count = hs;
    run(a);
  }
  return hipGetLastError();
}

}  // namespace la
