// Gated recurrence with a per-key-dimension decay and grouped query heads (the
// LinearAttention operator page, ai.onnx since version 27, "gated" update rule
// with decay of shape (B, T, kv_num_heads * d_k); its gated_perdim_decay
// example): per kv head and token,
//   S_t = diag(exp(g_t)) S_{t-1} + k_t v_t^T,   o_t = scale * q_t^T S_t,
// g_t a log-space vector over the key dimensions (rows of S).
//
// Chunk-parallel form over chunks of 64 tokens.  With b_t the inclusive
// cumulative decay inside the chunk (one value per key dim, b_{-1} = 0):
//   S_t  = diag(e^{b_t}) S_0 + sum_{s<=t} diag(e^{b_t - b_s}) k_s v_s^T
//   o_t  = scale * [ (q_t . e^{b_t})^T S_0 + sum_{s<=t} A_ts v_s ],
//   A_ts = sum_d q_td k_sd e^{b_td - b_sd}
//   S_C  = diag(e^{b_C}) S_0 + sum_s diag(e^{b_C - b_s}) k_s v_s^T  (C: last token).
// Decays are at most 1 (g <= 0), so q . e^{b_t}, e^{b_C} and e^{b_C - b_s} never
// exceed 1.  A is factorised per block of 32 keys sigma, with c_sigma = b at the
// token before the block (0 for the first):
//   A_ts = sum_d (q_td e^{b_td - c_sigma,d}) (k_sd e^{c_sigma,d - b_sd}),
// the query factor at most 1 (t is not before the block) and the key factor at
// least 1, bounded by the decay across the block's own 32 tokens: per-dim decays
// stronger than about 87 (log-space, summed over 32 tokens) overflow it.  The
// keys k^ = k e^{c - b} are formed once per chunk in LDS beside the raw keys,
// which the state update uses with e^{b_C - b_s} applied in fp32.  When some
// dimension's cumulative decay inside a chunk exceeds kExactSpan in magnitude
// (the factors could leave the fp32 range), the workgroup flags its segment,
// and a second launch re-evaluates the segment's outputs and state token by
// token (la_recur.hpp), which holds for decays of any strength.
//
// Workgroup shape, loaders, V^T staging (hi + lo tiles for fp16 inputs) and the
// MFMA operand conventions follow the per-head-decay kernel (la_gated.hip).
#include "la_device.hpp"
#include "la_launch.hpp"
#include "la_recur.hpp"

namespace la {

// Largest |cumulative log decay| inside a chunk (any dimension) for which the
// factorised products stay well inside the fp32 range (e^{60} ~ 1e26); beyond
// it the workgroup re-evaluates its outputs token by token.
constexpr float kExactSpan = 60.f;

template <int G>
struct PdShape {
  static constexpr int P = G >= 2 ? 2 : 1;  // head parts per workgroup
  static constexpr int NW = 4 * P;          // wavefronts
  static constexpr int NTH = 64 * NW;       // threads
  static constexpr int HPW = G / P;         // query heads per wave
};

// The state pass (no outputs) of bf16 inputs asks for two workgroups per CU
// (at most 128 registers); it keeps no rescaled keys, so its LDS allows it
// (fp16 inputs add the V lo tile, which does not fit twice).
template <typename IT, int G, int MODE>
struct PdOccupancy {
  static constexpr int value = (PdShape<G>::NW == 8 && MODE != kModeCausal && std::is_same_v<IT, uint16_t>) ? 4 : 1;
};

template <typename IT, int D, int G, int MODE>
__global__ __launch_bounds__(PdShape<G>::NTH, (PdOccupancy<IT, G, MODE>::value)) void gated_pd_kernel(GatedArgs a) {
  using DT = typename Io<IT>::DT;
  using O = Op<DT>;
  using SH = PdShape<G>;
  constexpr int P = SH::P, NW = SH::NW, NTH = SH::NTH, HPW = SH::HPW;
  constexpr int VEC = O::VEC, KB = O::KB, ESZ = O::ESZ;
  constexpr int NDT = D / 16;
  constexpr int CB = D / VEC;
  constexpr int LOADERS = (kChunk * CB / NTH >= 2 || ESZ == 4) ? (NTH < kChunk * CB ? NTH : kChunk * CB)
                                                                : kChunk * CB / 2;
  constexpr int NTOK = kChunk * CB / LOADERS;
  constexpr int TW = (64 / CB) * NTOK;  // tokens of one loader wave
  constexpr int NQ = D / KB;
  constexpr int NKS = kChunk / KB;
  constexpr int PADE = 16 / ESZ;
  constexpr int KN_LD = D + PADE;
  constexpr int VT_LD = kChunk;
  constexpr int SB_LD = D + PADE;
  constexpr int BC_LD = D + 4;  // fp32 rows of the cumulative decays
  constexpr bool OUT = MODE == kModeCausal;
  constexpr bool VLO = !std::is_same_v<IT, DT>;
  constexpr int KN_BYTES = kChunk * KN_LD * ESZ;
  // 16-bit operands: k^ is kept as hi + lo bf16 tiles and q^ as hi + lo
  // registers, and A = Kh qh + Kl qh + Kh ql (the rescaled operands are not
  // inputs, so a single rounding of each would double the error of A)
  constexpr bool ALO = ESZ == 2;
  // k^ feeds A only: the state pass keeps neither tile
  constexpr int KH_BYTES = OUT ? KN_BYTES : 0;
  constexpr int KL_BYTES = (ALO && OUT) ? KN_BYTES : 0;
  constexpr int VT_BYTES = D * VT_LD * ESZ;
  constexpr int VL_BYTES = VLO ? D * VT_LD * ESZ : 0;
  constexpr int SB_BYTES = OUT ? D * SB_LD * ESZ : 0;
  constexpr int BC_BYTES = kChunk * BC_LD * 4;
  constexpr int WT_BYTES = NW * D * 4;
  constexpr int NS = NDT * NDT;
  constexpr int TPW = (NS + NW - 1) / NW;
  static_assert(NTOK >= 1 && NQ >= 1 && CB <= 64 && 64 % CB == 0, "unsupported head size");
  static_assert(ESZ == 4 || NTOK % 2 == 0, "bf16 V^T writes pack token pairs");
  static_assert(32 % TW == 0, "whole loader waves cover tokens 0..31");
  static_assert(LOADERS % 64 == 0, "whole loader waves");
  constexpr int K2_BYTES = KN_BYTES + KH_BYTES;
  static_assert(K2_BYTES + KL_BYTES + VT_BYTES + VL_BYTES + SB_BYTES + BC_BYTES + WT_BYTES <= 160 * 1024,
                "LDS budget");

  constexpr int SMEM = K2_BYTES + VT_BYTES + SB_BYTES + VL_BYTES + BC_BYTES + WT_BYTES + KL_BYTES + 16;
  __shared__ __align__(16) unsigned char smem[SMEM];
  __shared__ int rerun_flag;  // some chunk's decays exceed kExactSpan
  DT* Kn = (DT*)smem;                   // k as loaded (operand type, or raw fp16)
  DT* Kh = (DT*)(smem + KN_BYTES);      // k^ = k e^{c_sigma - b} (operand type; outputs only)
  DT* Vt = (DT*)(smem + K2_BYTES);
  DT* Sb = (DT*)(smem + K2_BYTES + VT_BYTES);
  DT* Vl = (DT*)(smem + K2_BYTES + VT_BYTES + SB_BYTES);
  float* Bc = (float*)(smem + K2_BYTES + VT_BYTES + SB_BYTES + VL_BYTES);
  float* Wt = (float*)(smem + K2_BYTES + VT_BYTES + SB_BYTES + VL_BYTES + BC_BYTES);
  DT* Kl = (DT*)(smem + K2_BYTES + VT_BYTES + SB_BYTES + VL_BYTES + BC_BYTES + WT_BYTES);  // lo of k^

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves w and w + 4 share a SIMD: row blocks wr and 3 - wr even out the
  // causal work between SIMDs
  const int hp = w >> 2, wr = (w & 4) ? 3 - (w & 3) : (w & 3);
  int l = tid & 63, lr = l & 15, lg = l >> 4;
  // query-head group hg of hs (the group's heads are G of the kv head's G * hs)
  const int hs = a.hsplit > 1 ? a.hsplit : 1;
  const int hc = a.hg_count > 0 ? a.hg_count : hs;  // groups of this launch, from hg_first
  const int hg = a.hg_first + blockIdx.x % hc;
  const int bid = blockIdx.x / hc;
  const int u = bid / a.seg_count;
  const int s = a.seg_first + bid % a.seg_count;
  const int Hq = a.Hq, Hkv = a.Hkv, T = a.T;
  const int b = u / Hkv, j = u % Hkv;
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int c0 = s * a.seg_chunks;
  const int c1 = min(c0 + a.seg_chunks, nchunks);
  const int QS = Hq * D, KS = Hkv * D;  // token strides of q/out and of k/v/decay
  const IT* qb = (const IT*)a.q + (int64_t)b * T * QS + (int64_t)(j * G * hs + hg * G) * D;
  IT* ob = (IT*)a.out + (int64_t)b * T * QS + (int64_t)(j * G * hs + hg * G) * D;
  const IT* kb = (const IT*)a.k + (int64_t)b * T * KS + (int64_t)j * D;
  const IT* vb = (const IT*)a.v + (int64_t)b * T * KS + (int64_t)j * D;
  const IT* gb = (const IT*)a.decay + (int64_t)b * T * KS + (int64_t)j * D;
  const float scale = a.scale;
  auto vt_at = [&](int r, int blk) { return r * VT_LD + ((blk ^ vt_swz(r)) * VEC); };
  auto kn_at = [&](int t, int col) {
    return t * KN_LD + (((col / VEC) ^ (kn_swz(t) & (CB - 1))) * VEC) + (col % VEC);
  };
  auto sq_at = [&](int r, int col) {
    return r * SB_LD + (((col / VEC) ^ sq_swz(r)) * VEC) + (col % VEC);
  };

  if (tid == 0) rerun_flag = 0;  // (read only after the chunk loop's barriers)
  // ---- state tiles: wave w owns tiles tau = w*TPW + i (rows rt, columns ct)
  f32x4_t sacc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) sacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (OUT) {
    const float* sin = a.s_in ? a.s_in + u * a.s_in_u + s * a.s_in_s : nullptr;
    if (sin) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int tau = w * TPW + i;
        if (tau < NS) {
          const int rt = tau / NDT, ct = tau % NDT;
#pragma unroll
          for (int q = 0; q < 4; ++q) sacc[i][q] = sin[(16 * rt + 4 * lg + q) * D + 16 * ct + lr];
        }
      }
    }
  }
  // S -> LDS, transposed [dv][dk], operand type
  auto write_sb = [&]() {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tau = w * TPW + i;
      if (tau < NS) {
        const int rt = tau / NDT, ct = tau % NDT;
        DT* p = Sb + sq_at(16 * ct + lr, 16 * rt + 4 * lg);
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
  if constexpr (OUT) write_sb();

  // ---- loads of the chunk's k, v and decay rows (clamped to the last token;
  // tokens past the end are zeroed when staged)
  const int cb = tid % CB, tg = tid / CB;
  const bool loader = tid < LOADERS;
  u32x4_t pk[NTOK], pv[NTOK], pg[NTOK];
  auto prefetch = [&](int c) {
    if (!loader) return;
    const int tb = c * kChunk;
#pragma unroll
    for (int n = 0; n < NTOK; ++n) {
      const int tok = min(tb + tg * NTOK + n, T - 1);
      const int64_t off = (int64_t)tok * KS + cb * VEC;
      pk[n] = ld16(kb + off);
      pv[n] = ld16(vb + off);
      pg[n] = ld16(gb + off);
    }
  };

  auto write_vt = [&](DT* base, const u32x4_t (&src)[NTOK]) {
    const int t0 = tg * NTOK;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int r = cb * VEC + e;
      if constexpr (ESZ == 2) {
#pragma unroll
        for (int n = 0; n < NTOK; n += 2) {
          const uint32_t w0 = src[n][e >> 1], w1 = src[n + 1][e >> 1];
          *(uint32_t*)(base + vt_at(r, (t0 + n) / VEC) + (t0 + n) % VEC) =
              (e & 1) ? __builtin_amdgcn_perm(w1, w0, 0x07060302u) : __builtin_amdgcn_perm(w1, w0, 0x05040100u);
        }
      } else {
        float fv[NTOK];
#pragma unroll
        for (int n = 0; n < NTOK; ++n) fv[n] = __uint_as_float(src[n][e]);
        DT* p = base + vt_at(r, t0 / VEC) + (t0 % VEC);
        if constexpr (NTOK == 1) {
          *(float*)p = fv[0];
        } else if constexpr (NTOK == 2) {
          *(float2*)p = make_float2(fv[0], fv[1]);
        } else {
#pragma unroll
          for (int n = 0; n < NTOK; n += 4)
            *(f32x4_t*)(base + vt_at(r, (t0 + n) / VEC)) = f32x4_t{fv[n], fv[n + 1], fv[n + 2], fv[n + 3]};
        }
      }
    }
  };

  // ---- stage: raw k -> Kn, V -> V^T (+ lo), per-dim inclusive scan of the
  // decays -> Bc, k^ -> Kh.  Ends with the chunk's LDS complete (barrier).
  auto stage = [&](int c) {
    const int tb = c * kChunk;
    float bx[NTOK][VEC];   // the loader's cumulative decays (tokens n, dims cb*VEC + e)
    float tot[VEC];        // their wave-exclusive offset, then the wave total
    if (loader) {
      if (tb + kChunk > T) {
#pragma unroll
        for (int n = 0; n < NTOK; ++n)
          if (tb + tg * NTOK + n >= T) {
            pk[n] = u32x4_t{0u, 0u, 0u, 0u};
            pv[n] = u32x4_t{0u, 0u, 0u, 0u};
            pg[n] = u32x4_t{0u, 0u, 0u, 0u};
          }
      }
#pragma unroll
      for (int n = 0; n < NTOK; ++n) st16(Kn + kn_at(tg * NTOK + n, cb * VEC), pk[n]);
#pragma unroll
      for (int n = 0; n < NTOK; ++n) Io<IT>::unpack(pg[n], bx[n]);
      if constexpr (VLO) {
        u32x4_t pl[NTOK];
#pragma unroll
        for (int n = 0; n < NTOK; ++n) {
          float f[VEC];
          Io<IT>::unpack(pv[n], f);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t hw = pack_bf16x2(f[2 * i], f[2 * i + 1]);
            pv[n][i] = hw;
            pl[n][i] = pack_bf16x2(f[2 * i] - __uint_as_float(hw << 16),
                                   f[2 * i + 1] - __uint_as_float(hw & 0xffff0000u));
          }
        }
        write_vt(Vl, pl);
      }
      write_vt(Vt, pv);
      // scan over the thread's own tokens, then across the wave's lanes with
      // the same dims (lanes cb, cb + CB, ...: consecutive token groups)
#pragma unroll
      for (int n = 1; n < NTOK; ++n)
#pragma unroll
        for (int e = 0; e < VEC; ++e) bx[n][e] += bx[n - 1][e];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float x = bx[NTOK - 1][e];
        const float own = x;
#pragma unroll
        for (int k = CB; k < 64; k <<= 1) {
          const float y = __shfl_up(x, k);
          if (l >= k) x += y;
        }
        tot[e] = x - own;  // exclusive offset inside the wave
        if (l >= 64 - CB) Wt[w * D + cb * VEC + e] = x;  // the wave's total for this dim
      }
    }
    __syncthreads();
    if (loader) {
      // offsets of the earlier loader waves, and c_32 = b at token 31
      float off[VEC], c32[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        off[e] = tot[e];
        c32[e] = 0.f;
      }
      for (int w2 = 0; w2 < w; ++w2) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) off[e] += Wt[w2 * D + cb * VEC + e];
      }
      constexpr int W32 = 32 / TW;  // loader waves covering tokens 0..31
#pragma unroll
      for (int w2 = 0; w2 < W32; ++w2)
#pragma unroll
        for (int e = 0; e < VEC; ++e) c32[e] += Wt[w2 * D + cb * VEC + e];
      float span = 0.f;
#pragma unroll
      for (int n = 0; n < NTOK; ++n) {
        const int t = tg * NTOK + n;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          bx[n][e] += off[e];
          span = fmaxf(span, fabsf(bx[n][e]));
        }
#pragma unroll
        for (int e = 0; e < VEC; e += 4)
          *(f32x4_t*)(Bc + t * BC_LD + cb * VEC + e) = f32x4_t{bx[n][e], bx[n][e + 1], bx[n][e + 2], bx[n][e + 3]};
      }
      if (OUT && !(span <= kExactSpan)) rerun_flag = 1;  // (NaN decays too)
#pragma unroll
      for (int n = 0; n < NTOK && OUT; ++n) {
        const int t = tg * NTOK + n;
        float kx[VEC];
        Io<IT>::unpack(pk[n], kx);
        float kh[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float cs = t >= 32 ? c32[e] : 0.f;
          kh[e] = kx[e] * __expf(cs - bx[n][e]);
        }
        const u32x4_t hi = O::pack(kh);
        st16(Kh + kn_at(t, cb * VEC), hi);
        if constexpr (ALO) {
          float kl[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) kl[e] = kh[e] - bf16_bits_to_f32((hi[e >> 1] >> (16 * (e & 1))) & 0xffffu);
          st16(Kl + kn_at(t, cb * VEC), O::pack(kl));
        }
      }
    }
    __syncthreads();
  };

  float seg_log = 0.f;  // state mode: thread tid < D sums b_C of dim tid

  auto compute = [&](int c) {
    if constexpr (!OUT) {
      // the state pass re-derives its lane indices per chunk (opaque_lane):
      // the addresses built from them are not held across the loop, which
      // keeps it within two workgroups' registers
      l = opaque_lane(tid);
      lr = l & 15;
      lg = l >> 4;
    }
    const int tq = 16 * wr + lr;  // the lane's query row in the chunk
    if constexpr (OUT) {
      const int tok = c * kChunk + tq;
      const int tokc = min(tok, T - 1);
      // keys of A^T tile t (bf16: tile pairs over 32 keys with permuted rows;
      // fp32: 16-key tiles), and whether the wave's queries need it
      auto key_of = [&](int t, int q) {
        return ESZ == 2 ? 32 * (t >> 1) + 8 * lg + 4 * (t & 1) + q : 16 * t + 4 * lg + q;
      };
      auto need = [&](int t) { return ESZ == 2 ? (32 * (t >> 1) <= 16 * wr + 15) : (t <= wr); };
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const int hq = hp + P * hh;
        // q of row tq in operand layout (dims KB*m + VEC*lg + e), as loaded
        u32x4_t qr[NQ];
#pragma unroll
        for (int m = 0; m < NQ; ++m) qr[m] = ld16(qb + (int64_t)tokc * QS + hq * D + KB * m + VEC * lg);
        // q . e^{b_t - c}: block 0 (c = 0, also the inter-chunk factor) and block 1 (c = b_31)
        auto qhat = [&](u32x4_t (&dst)[NQ], u32x4_t (&dlo)[ALO ? NQ : 1], bool second) {
          // the factors are the same for every head; the row offsets pass
          // through an empty asm so that each head recomputes them instead of
          // keeping all of them live across the heads
          int rt_off = tq * BC_LD, r31_off = 31 * BC_LD;
          asm volatile("" : "+v"(rt_off), "+v"(r31_off));
#pragma unroll
          for (int m = 0; m < NQ; ++m) {
            const int d0 = KB * m + VEC * lg;
            float f[VEC];
            Io<IT>::unpack(qr[m], f);
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
              const f32x4_t bt = *(const f32x4_t*)(Bc + rt_off + d0 + e);
              f32x4_t cs = f32x4_t{0.f, 0.f, 0.f, 0.f};
              if (second) cs = *(const f32x4_t*)(Bc + r31_off + d0 + e);
#pragma unroll
              for (int i = 0; i < 4; ++i) f[e + i] *= __expf(bt[i] - cs[i]);
            }
            dst[m] = O::pack(f);
            if constexpr (ALO) {
              float r[VEC];
#pragma unroll
              for (int e = 0; e < VEC; ++e)
                r[e] = f[e] - bf16_bits_to_f32((dst[m][e >> 1] >> (16 * (e & 1))) & 0xffffu);
              dlo[m] = O::pack(r);
            }
          }
        };
        // decayed, causally masked A^T tile t from k^ rows and the block's q^
        auto a_tile = [&](int t, const u32x4_t (&qh)[NQ], const u32x4_t (&ql)[ALO ? NQ : 1]) {
          f32x4_t at = f32x4_t{0.f, 0.f, 0.f, 0.f};
          const int krow = ESZ == 2 ? 32 * (t >> 1) + 8 * (lr >> 2) + 4 * (t & 1) + (lr & 3) : 16 * t + lr;
#pragma unroll
          for (int m = 0; m < NQ; ++m) {
            const u32x4_t kh = ld16(Kh + kn_at(krow, KB * m + VEC * lg));
            O::mma(at, kh, qh[m]);
            if constexpr (ALO) {
              O::mma(at, ld16(Kl + kn_at(krow, KB * m + VEC * lg)), qh[m]);
              O::mma(at, kh, ql[m]);
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) at[q] = key_of(t, q) <= tq ? at[q] : 0.f;
          return at;
        };
        u32x4_t qop[NQ], qlo[ALO ? NQ : 1];
        qhat(qop, qlo, false);
        // the first key block's tiles before the inter-chunk product (its q^ lo
        // then dies early)
        f32x4_t a0[2];
        a0[0] = a_tile(0, qop, qlo);
        a0[1] = need(1) ? a_tile(1, qop, qlo) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        f32x4_t nacc[NDT];
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) nacc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // inter-chunk: S_0^T (q . e^{b_t})
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
#pragma unroll
          for (int ct = 0; ct < NDT; ++ct) {
            const u32x4_t av = ld16(Sb + sq_at(16 * ct + lr, KB * m + VEC * lg));
            O::mma(nacc[ct], av, qop[m]);
          }
        }
        if constexpr (ESZ == 2) {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            if (need(2 * p)) {
              f32x4_t at0 = a0[0], at1 = a0[1];
              if (p == 1) {
                qhat(qop, qlo, true);
                at0 = a_tile(2, qop, qlo);
                at1 = a_tile(3, qop, qlo);
              }
              u32x4_t bh, bl;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const f32x4_t& at = (e >> 1) ? at1 : at0;
                const float x0 = at[2 * (e & 1)], x1 = at[2 * (e & 1) + 1];
                const uint32_t hw = pack_bf16x2(x0, x1);
                bh[e] = hw;
                bl[e] = pack_bf16x2(x0 - __uint_as_float(hw << 16), x1 - __uint_as_float(hw & 0xffff0000u));
              }
#pragma unroll
              for (int ct = 0; ct < NDT; ++ct) {
                const u32x4_t av = ld16(Vt + vt_at(16 * ct + lr, 4 * p + lg));
                O::mma(nacc[ct], av, bh);
                O::mma(nacc[ct], av, bl);
                if constexpr (VLO) O::mma(nacc[ct], ld16(Vl + vt_at(16 * ct + lr, 4 * p + lg)), bh);
              }
            }
          }
        } else {
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) {
            if (need(jt)) {
              if (jt == 2) qhat(qop, qlo, true);
              const f32x4_t at = jt < 2 ? a0[jt] : a_tile(jt, qop, qlo);
#pragma unroll
              for (int ct = 0; ct < NDT; ++ct) {
                const u32x4_t av = ld16(Vt + vt_at(16 * ct + lr, 4 * jt + lg));
#pragma unroll
                for (int q = 0; q < 4; ++q)
                  nacc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av[q]), at[q], nacc[ct], 0, 0, 0);
              }
            }
          }
        }
        if (tok < T) {
          IT* orow = ob + (int64_t)tok * QS + hq * D + 4 * lg;
#pragma unroll
          for (int ct = 0; ct < NDT; ++ct)
            store4(orow + 16 * ct, scale * nacc[ct][0], scale * nacc[ct][1], scale * nacc[ct][2],
                   scale * nacc[ct][3]);
        }
      }
    }
    // ---- state: S = diag(e^{b_C}) S + sum_s diag(e^{b_C - b_s}) k_s v_s^T, with
    // the raw keys, the factors in fp32 and the decayed keys as hi + lo
    // the chunk's last token (the sequence's last in a partial chunk: its
    // cumulative decay is then exactly the newest token's, whatever order the
    // scan summed the padded zeros in)
    const int cl = min(kChunk, T - c * kChunk) - 1;
    if constexpr (!OUT) {
      if (tid < D) seg_log += Bc[cl * BC_LD + tid];
    }
    u32x4_t kop[NKS], kol[NKS];
    float er[4];  // the chunk's decay of state rows 16 rt + 4 lg + q (the same for a row tile's column tiles)
    int cur_rt = -1;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tau = w * TPW + i;
      if (tau < NS) {
        const int rt = tau / NDT, ct = tau % NDT;
        if (rt != cur_rt) {
          cur_rt = rt;
#pragma unroll
          for (int q = 0; q < 4; ++q) er[q] = __expf(Bc[cl * BC_LD + 16 * rt + 4 * lg + q]);
          const int dk = 16 * rt + lr;
          const float bC = Bc[cl * BC_LD + dk];
#pragma unroll
          for (int m = 0; m < NKS; ++m) {
            float f[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              const int sk = KB * m + VEC * lg + e;
              const float kw = __expf(bC - Bc[sk * BC_LD + dk]);
              const int off = kn_at(sk, dk);
              if constexpr (ESZ == 2)
                f[e] = Io<IT>::to_f32(((const uint16_t*)Kn)[off]) * kw;
              else
                f[e] = ((const float*)Kn)[off] * kw;
            }
            kop[m] = O::pack(f);
            if constexpr (ESZ == 2) {
              float r[VEC];
#pragma unroll
              for (int e = 0; e < VEC; ++e) {
                const uint32_t hb = (kop[m][e >> 1] >> (16 * (e & 1))) & 0xffffu;
                r[e] = f[e] - bf16_bits_to_f32(hb);
              }
              kol[m] = O::pack(r);
            }
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) sacc[i][q] *= er[q];
#pragma unroll
        for (int m = 0; m < NKS; ++m) {
          const u32x4_t bv = ld16(Vt + vt_at(16 * ct + lr, (KB / VEC) * m + lg));
          O::mma(sacc[i], kop[m], bv);
          if constexpr (ESZ == 2) O::mma(sacc[i], kol[m], bv);
          if constexpr (VLO) O::mma(sacc[i], kop[m], ld16(Vl + vt_at(16 * ct + lr, (KB / VEC) * m + lg)));
        }
      }
    }
  };

  if (c0 < c1) prefetch(c0);
  for (int c = c0; c < c1; ++c) {
    stage(c);
    prefetch(min(c + 1, c1 - 1));
    compute(c);
    __syncthreads();
    if constexpr (OUT) write_sb();
  }

  float* sout = nullptr;
  if constexpr (OUT) {
    if (s == a.nseg_total - 1 && hg == 0) sout = a.s_out + u * a.s_out_u;
  } else {
    sout = a.s_out + u * a.s_out_u + (s + a.out_slot_off) * a.s_out_s;
    if (tid < D) a.a_out[((int64_t)u * a.nseg_total + s + a.out_slot_off) * D + tid] = __expf(seg_log);
  }
  // (a flagged segment's state is stored by the re-evaluation: stored here,
  // it would overwrite a start state the re-evaluation reads when the state is
  // updated in place)
  if (sout && !(OUT && rerun_flag)) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tau = w * TPW + i;
      if (tau < NS) {
        const int rt = tau / NDT, ct = tau % NDT;
#pragma unroll
        for (int q = 0; q < 4; ++q) sout[(16 * rt + 4 * lg + q) * D + 16 * ct + lr] = sacc[i][q];
      }
    }
  }
  if constexpr (OUT) {
    // (all query-head groups see the same decays: group 0 stores the flag)
    if (tid == 0 && hg == 0) a.flags[u * a.nseg_total + s] = rerun_flag;
  }
}

// Strong decays: the segments whose output pass set their flag, outputs and
// final state again token by token (la_recur.hpp), which holds for decays of
// any strength.  Same grid, query-head groups and pointers as the output pass;
// the others return at once.  The re-evaluation lives in a launch of its own:
// inside the output kernel its code cost that kernel about 7% on the per-dim
// workload, though it rarely runs.
template <typename IT, int D, int G>
__global__ __launch_bounds__(PdShape<G>::NTH) void gated_pd_rerun_kernel(GatedArgs a) {
  constexpr int NTH = PdShape<G>::NTH;
  constexpr int RHP = recur_heads<D, NTH, G>(128 * 1024);  // heads per pass
  static_assert(RHP >= 1, "LDS for the token-by-token re-evaluation");
  __shared__ __align__(16) unsigned char smem[recur_lds_bytes<D, NTH, G, RHP>()];
  const int hs = a.hsplit > 1 ? a.hsplit : 1;
  const int hc = a.hg_count > 0 ? a.hg_count : hs;
  const int hg = a.hg_first + blockIdx.x % hc;
  const int bid = blockIdx.x / hc;
  const int u = bid / a.seg_count;
  const int s = a.seg_first + bid % a.seg_count;
  if (!a.flags[u * a.nseg_total + s]) return;
  const int Hq = a.Hq, Hkv = a.Hkv, T = a.T;
  const int b = u / Hkv, j = u % Hkv;
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int c0 = s * a.seg_chunks;
  const int c1 = min(c0 + a.seg_chunks, nchunks);
  const int QS = Hq * D, KS = Hkv * D;
  const int64_t qo = (int64_t)b * T * QS + (int64_t)(j * G * hs + hg * G) * D;
  const int64_t ko = (int64_t)b * T * KS + (int64_t)j * D;
  RecurPtrs rp;
  rp.q = (const IT*)a.q + qo;
  rp.k = (const IT*)a.k + ko;
  rp.v = (const IT*)a.v + ko;
  rp.decay = (const IT*)a.decay + ko;
  rp.beta = nullptr;
  rp.out = (IT*)a.out + qo;
  rp.s_in = a.s_in ? a.s_in + u * a.s_in_u + s * a.s_in_s : nullptr;
  rp.s_out = (s == a.nseg_total - 1 && hg == 0) ? a.s_out + u * a.s_out_u : nullptr;
  rp.qs = QS;
  rp.ks = KS;
  rp.gs = KS;
  rp.bs = 0;
  rp.t0 = c0 * kChunk;
  rp.t1 = min(c1 * kChunk, T);
  rp.scale = a.scale;
  token_recurrence<IT, D, NTH, G, RHP, 2, false>(smem, rp);
}

template <typename IT, int D, int G>
static hipError_t launch_pg(int mode, const GatedArgs& a, int grid, hipStream_t st) {
  constexpr int NTH = PdShape<G>::NTH;
  if (mode == kModeCausal)
    hipLaunchKernelGGL((gated_pd_kernel<IT, D, G, kModeCausal>), dim3(grid), dim3(NTH), 0, st, a);
  else if (mode == kModeRerun)
    hipLaunchKernelGGL((gated_pd_rerun_kernel<IT, D, G>), dim3(grid), dim3(NTH), 0, st, a);
  else
    hipLaunchKernelGGL((gated_pd_kernel<IT, D, G, kModeState>), dim3(grid), dim3(NTH), 0, st, a);
  return hipGetLastError();
}

template <typename IT, int D>
static hipError_t launch_pgd(int mode, int G, const GatedArgs& a, int grid, hipStream_t st) {
  switch (G) {
    case 1: return launch_pg<IT, D, 1>(mode, a, grid, st);
    case 2: return launch_pg<IT, D, 2>(mode, a, grid, st);
    case 4: return launch_pg<IT, D, 4>(mode, a, grid, st);
    default: return launch_pg<IT, D, 8>(mode, a, grid, st);
  }
}

template <typename IT>
static hipError_t launch_pgdt(int mode, int D, int G, const GatedArgs& a, int grid, hipStream_t st) {
  switch (D) {
    case 32: return launch_pgd<IT, 32>(mode, G, a, grid, st);
    case 64: return launch_pgd<IT, 64>(mode, G, a, grid, st);
    default:
      if constexpr (sizeof(IT) == 2) return launch_pgd<IT, 128>(mode, G, a, grid, st);
      return hipErrorInvalidValue;  // fp32 at head size 128 does not fit LDS
  }
}

hipError_t launch_gated_pd(int mode, int io, int D, int G, const GatedArgs& a, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  switch (io) {
    case kIoBF16: return launch_pgdt<uint16_t>(mode, D, G, a, grid, st);
    case kIoF16: return launch_pgdt<f16_t>(mode, D, G, a, grid, st);
    default: return launch_pgdt<float>(mode, D, G, a, grid, st);
  }
}

}  // namespace la
