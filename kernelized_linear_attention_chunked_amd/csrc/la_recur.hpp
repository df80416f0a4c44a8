// Token-by-token evaluation of one (batch, kv head) unit of the gated and
// delta recurrences (the LinearAttention operator page, ai.onnx since version
// 27, "Description": S_t = E_t S_{t-1} + k_t v_t^T for "gated", and
// S_t = E_t S_{t-1} + beta_t k_t (v_t - (E_t S_{t-1})^T k_t)^T for
// "gated_delta"; o_t = scale q_t^T S_t per query head).
//
// The chunk kernels factorise the in-chunk decay into per-row and per-key
// factors relative to a reference token, which leaves the fp32 range when a
// dimension's decay over a chunk is very strong.  A workgroup that meets such
// a chunk re-evaluates its tokens with this routine, which applies exp(g_t)
// one token at a time (every factor at most 1 for g <= 0) and so holds for
// decays of any strength.  It is slow (a few barriers per token) and runs only
// for those workgroups.
//
// Layout: of the NTH threads, the first NTS = min(NTH, D * D / 4) hold the
// state: thread (c4, rg) holds columns 4*c4 .. 4*c4+3 of state rows rg + RG*r
// (r < RPT) in registers.  The readouts of the GW query heads are summed over
// the row groups through LDS, HP heads per pass.
#pragma once

#include "la_device.hpp"

namespace la {

struct RecurPtrs {
  const void* q;      // query head 0 of the group at token t: q + t * qs (+ h * D)
  const void* k;      // k + t * ks
  const void* v;      // v + t * ks, or null (values zero)
  const void* decay;  // null, or g + t * gs (one value, or D values per token)
  const void* beta;   // delta rule only: beta + t * bs
  void* out;          // like q, or null (no outputs)
  const float* s_in;  // D x D initial state or null (zeros)
  float* s_out;       // D x D final state or null (not written)
  int64_t qs, ks, gs, bs;
  int t0, t1;
  float scale;
};

// Bytes of LDS the routine needs for these sizes.
template <int D, int NTH>
struct RecurShape {
  static constexpr int C4 = D / 4;                           // float4 columns of a row
  static constexpr int NTS = NTH < D * C4 ? NTH : D * C4;    // threads holding the state
  static constexpr int RG = NTS / C4;                        // row groups
  static constexpr int RPT = D / RG;                         // rows per thread
};

template <int D, int NTH, int GW, int HP>
constexpr int recur_lds_bytes() {
  return (4 * D + GW * D + HP * RecurShape<D, NTH>::RG * D) * 4;
}

// The largest power-of-two count of query heads per readout pass (dividing
// GW) whose LDS fits in `avail` bytes; 0 if not even one head fits.
template <int D, int NTH, int GW>
constexpr int recur_heads(int avail) {
  for (int hp = GW; hp >= 1; hp /= 2)
    if (GW % hp == 0 && (4 * D + GW * D + hp * RecurShape<D, NTH>::RG * D) * 4 <= avail) return hp;
  return 0;
}

// DK: 0 no decay, 1 one per kv head, 2 one per key dimension.  DELTA: the
// delta rule (beta required).  GW: query heads of the workgroup; HP: heads per
// readout pass (GW % HP == 0).  `lds`: recur_lds_bytes<D, NTH, GW, HP>() bytes,
// not in use by anything else.  Every thread of the workgroup must call it.
template <typename IT, int D, int NTH, int GW, int HP, int DK, bool DELTA>
__device__ void token_recurrence(unsigned char* lds, const RecurPtrs& r) {
  using RS = RecurShape<D, NTH>;
  constexpr int C4 = RS::C4, NTS = RS::NTS, RG = RS::RG, RPT = RS::RPT;
  static_assert(RG * C4 == NTS && RPT * RG == D && GW % HP == 0, "unsupported shape");
  float* fk = (float*)lds;      // k_t
  float* fv = fk + D;           // v_t
  float* fe = fv + D;           // exp(g_t) per row (DK == 2) or in fe[0]
  float* fw = fe + D;           // delta: beta (v - S'^T k)
  float* fq = fw + D;           // [GW][D] queries
  float* part = fq + GW * D;    // [HP][RG][D] partial readouts
  const int tid = threadIdx.x;
  const bool holder = tid < NTS;  // holds state rows
  const int c4 = tid % C4, rg = (tid / C4) % RG;
  const IT* qb = (const IT*)r.q;
  const IT* kb = (const IT*)r.k;
  const IT* vb = (const IT*)r.v;
  const IT* gb = (const IT*)r.decay;
  const IT* bb = (const IT*)r.beta;
  IT* ob = (IT*)r.out;
  auto ld = [](const IT* p, int64_t i) { return Io<IT>::to_f32(sizeof(IT) == 4 ? __float_as_uint(((const float*)p)[i])
                                                                               : (uint32_t)((const uint16_t*)p)[i]); };

  static_assert(D <= NTH, "one thread per key dimension");
  f32x4_t sv[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    sv[i] = (r.s_in && holder) ? *(const f32x4_t*)(r.s_in + (rg + RG * i) * D + 4 * c4) : f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the next token's inputs are loaded into registers while the current one
  // is processed: thread i < D takes k, v (and a per-dim decay) of dimension i,
  // every thread NQE query elements
  constexpr int NQE = (GW * D + NTH - 1) / NTH;
  float pk = 0.f, pv = 0.f, pg = 0.f, pb = 0.f, pq[NQE];
  auto fetch = [&](int t) {
    if (tid < D) {
      pk = ld(kb + (int64_t)t * r.ks, tid);
      pv = vb ? ld(vb + (int64_t)t * r.ks, tid) : 0.f;
      if constexpr (DK == 2) pg = ld(gb + (int64_t)t * r.gs, tid);
    }
    if constexpr (DK == 1) pg = ld(gb + (int64_t)t * r.gs, 0);
    if constexpr (DELTA) pb = ld(bb + (int64_t)t * r.bs, 0);
#pragma unroll
    for (int j = 0; j < NQE; ++j) {
      const int i = tid + j * NTH;
      pq[j] = i < GW * D ? ld(qb + (int64_t)t * r.qs, i) : 0.f;
    }
  };
  if (r.t0 < r.t1) fetch(r.t0);

  for (int t = r.t0; t < r.t1; ++t) {
    if (tid < D) {
      fk[tid] = pk;
      fv[tid] = pv;
      if constexpr (DK == 2) fe[tid] = __expf(pg);
    }
    if constexpr (DK == 1)
      if (tid == 0) fe[0] = __expf(pg);
    const float be = pb;
#pragma unroll
    for (int j = 0; j < NQE; ++j) {
      const int i = tid + j * NTH;
      if (i < GW * D) fq[i] = pq[j];
    }
    if (t + 1 < r.t1) fetch(t + 1);
    __syncthreads();
    // S' = E S
    if (DK != 0 && holder) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float e = DK == 2 ? fe[rg + RG * i] : fe[0];
#pragma unroll
        for (int c = 0; c < 4; ++c) sv[i][c] *= e;
      }
    }
    if constexpr (DELTA) {
      // w = S'^T k summed over the row groups, then u = beta (v - w)
      if (holder) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const float kd = fk[rg + RG * i];
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] = fmaf(kd, sv[i][c], acc[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) part[rg * D + 4 * c4 + c] = acc[c];
      }
      __syncthreads();
      for (int i = tid; i < D; i += NTH) {
        float wsum = 0.f;
        for (int g = 0; g < RG; ++g) wsum += part[g * D + i];
        fw[i] = be * (fv[i] - wsum);
      }
      __syncthreads();
    }
    // S'' = S' + k u^T (u = v for the gated rule)
    const float* uu = DELTA ? fw : fv;
    if (holder) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float kd = fk[rg + RG * i];
#pragma unroll
        for (int c = 0; c < 4; ++c) sv[i][c] = fmaf(kd, uu[4 * c4 + c], sv[i][c]);
      }
    }
    // o_h = scale q_h^T S'', HP heads per pass (none without outputs)
    for (int h0 = 0; ob && h0 < GW; h0 += HP) {
#pragma unroll
      for (int h = 0; h < HP && holder; ++h) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const float qd = fq[(h0 + h) * D + rg + RG * i];
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] = fmaf(qd, sv[i][c], acc[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) part[(h * RG + rg) * D + 4 * c4 + c] = acc[c];
      }
      __syncthreads();
      for (int i = tid; i < HP * D; i += NTH) {
        const int h = i / D, d = i % D;
        float y = 0.f;
        for (int g = 0; g < RG; ++g) y += part[(h * RG + g) * D + d];
        y *= r.scale;
        IT* op = ob + (int64_t)t * r.qs + (int64_t)(h0 + h) * D + d;
        if constexpr (std::is_same_v<IT, uint16_t>)
          *op = (uint16_t)f32_to_bf16_bits(y);
        else
          *op = (IT)y;
      }
      __syncthreads();
    }
  }
  if (r.s_out && holder) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) *(f32x4_t*)(r.s_out + (rg + RG * i) * D + 4 * c4) = sv[i];
  }
}

}  // namespace la
