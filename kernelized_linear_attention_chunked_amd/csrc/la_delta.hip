// Delta-rule recurrences with grouped query heads (the LinearAttention operator
// page, ai.onnx since version 27, update rules "delta" and "gated_delta"): per
// kv head and token,
//   S_t = D_t S_{t-1} + beta_t k_t (v_t - (D_t S_{t-1})^T k_t)^T,   o_t = scale q_t^T S_t,
// with D_t = I ("delta"), or diag(exp(g_t)) for a log-space decay g_t given per
// kv head or per key dimension ("gated_delta"), and beta_t per kv head or
// shared by all heads.
//
// Chunk-parallel form over chunks of 64 tokens (the delta rule's WY-style
// chunking).  With b_t the inclusive cumulative decay inside the chunk (per key
// dim; 0 without a decay), G_t = diag(e^{b_t}) and S_0 the state before it:
//   S_t = G_t X_t,  X_t = X_{t-1} + (G_t^-1 k_t) u_t^T,  X_{-1} = S_0,
//   u_t = beta_t (v_t - S_0^T (G_t k_t) - sum_{j<t} L_tj u_j),
//   L_tj = sum_d k_td k_jd e^{b_td - b_jd}          (j < t),
// which follows from substituting S_t = G_t X_t into the recurrence.  So the
// pseudo-values U solve the unit lower-triangular system
//   (I + diag(beta) L) U = diag(beta) (V - Kbar S_0),   Kbar = rows k_t e^{b_t},
// and then, exactly as for the per-dim gated rule with U in place of V,
//   o_t  = scale [ (q_t . e^{b_t})^T S_0 + sum_{j<=t} A_tj u_j ],
//   A_tj = sum_d q_td k_jd e^{b_td - b_jd},
//   S_C  = diag(e^{b_C}) S_0 + sum_j diag(e^{b_C - b_j}) k_j u_j^T.
// L and A use the per-dim kernel's block-relative rescaling of the keys
// (la_gated_pd.hip), with hi + lo bf16 operands for 16-bit inputs.
//
// The system is solved in four blocks of 16 rows, one after the other: the
// waves of row block i subtract the earlier blocks' contributions with MFMAs
// over U (hi + lo), then run a forward substitution over their own 16 rows in
// registers (lane shuffles), and write their rows of U^T over the V^T tiles.
// A sequence is processed by one workgroup from start to end, or split into
// segments when there are few (batch, kv head) units: a segment maps its
// start state affinely, S_end = M S_start + N, with M = prod_t (I - beta_t k_t
// k_t^T) D_t a full D x D matrix.  The same kernel runs each segment from
// S = I with zero values (M) and from S = 0 (N), without outputs; the start
// states follow by composing the maps in order (delta_compose_kernel), and
// every segment then runs again from its start state with outputs.
//
// The rescaled keys (per-dim decays, and fp16 inputs with a per-head decay)
// leave the fp32 range when a cumulative decay inside a chunk is very strong.
// A workgroup that meets a chunk whose |b| exceeds kDeltaExactSpan in some
// dimension re-evaluates its whole sequence token by token (la_recur.hpp),
// outputs and state, which holds for decays of any strength.
#include "la_device.hpp"
#include "la_launch.hpp"
#include "la_recur.hpp"

namespace la {

// Largest |cumulative log decay| inside a chunk for which the rescaled keys
// stay well inside the fp32 range (e^{60} ~ 1e26).
constexpr float kDeltaExactSpan = 60.f;

template <int G>
struct DeltaShape {
  static constexpr int P = G >= 2 ? 2 : 1;  // head parts (and dv halves) per workgroup
  static constexpr int NW = 4 * P;          // wavefronts
  static constexpr int NTH = 64 * NW;       // threads
  static constexpr int HPW = G / P;         // query heads per wave
};

// DK: 0 no decay ("delta"), 1 one decay per kv head, 2 one per key dimension.
template <typename IT, int D, int G, int DK>
__global__ __launch_bounds__(DeltaShape<G>::NTH) void delta_kernel(DeltaArgs a) {
  using DT = typename Io<IT>::DT;
  using O = Op<DT>;
  using SH = DeltaShape<G>;
  constexpr int P = SH::P, NW = SH::NW, NTH = SH::NTH, HPW = SH::HPW;
  constexpr int VEC = O::VEC, KB = O::KB, ESZ = O::ESZ;
  constexpr int NDT = D / 16;
  constexpr int RH = NDT / P;  // dv tiles of a wave in the solve
  constexpr int CB = D / VEC;
  constexpr int LOADERS = (kChunk * CB / NTH >= 2 || ESZ == 4) ? (NTH < kChunk * CB ? NTH : kChunk * CB)
                                                                : kChunk * CB / 2;
  constexpr int NTOK = kChunk * CB / LOADERS;
  constexpr int TW = (64 / CB) * NTOK;  // tokens of one loader wave
  constexpr int NQ = D / KB;
  constexpr int NKS = kChunk / KB;
  // 16-bit operands: unpadded rows with the swizzles ksw / qsw (la_device.hpp)
  constexpr bool SWZ = ESZ == 2;
  constexpr int PADE = SWZ ? 0 : 16 / ESZ;
  constexpr int KN_LD = D + PADE;
  constexpr int VT_LD = kChunk;
  constexpr int SB_LD = D + PADE;
  constexpr int BC_LD = D + 4;
  constexpr bool LO = ESZ == 2;   // 16-bit: hi + lo operands (k^, q^, U, L, A)
  // RAW: bf16 or fp32 inputs without a per-dim decay.  q and k then enter the
  // MFMAs as they are (exact), and a per-head decay is applied in fp32 after
  // each product: exp(b_t - b_j) per element of A and L, exp(b_t) per row of
  // the inter term and of Kbar S_0, as in the per-head gated kernel; no factor
  // exceeds 1 for decays <= 0.  Otherwise (fp16 inputs, per-dim decays) the
  // scaled rows q^, kbar and the keys k^ are formed first relative to 32-token
  // blocks, and carry a lo part.
  constexpr bool RAW = DK <= 1 && (std::is_same_v<IT, uint16_t> || std::is_same_v<IT, float>);
  constexpr bool XLO = LO && !RAW;
  constexpr bool RAWDEC = RAW && DK == 1;  // RAW with factors to apply
  // RAW bf16 with an even number of query heads per wave: outputs by head pairs
  constexpr bool PAIR = RAW && ESZ == 2 && HPW % 2 == 0;
  constexpr int KN_BYTES = kChunk * KN_LD * ESZ;
  constexpr int VT_BYTES = D * VT_LD * ESZ;
  constexpr int SB_BYTES = D * SB_LD * ESZ;
  // the per-dim decay table only for per-dim decays; without it, the LDS holds
  // a lo part of S (16-bit), used where S_0 meets the state (R) and the outputs
  constexpr int BC_BYTES = DK == 2 ? kChunk * BC_LD * 4 : 0;
  constexpr bool SLO = LO && DK != 2;
  constexpr int SL_BYTES = SLO ? SB_BYTES : 0;
  constexpr int WT_BYTES = NW * D * 4;
  constexpr int BT_BYTES = 2 * kChunk * 4;  // beta and the per-head cumulative decay
  constexpr int LB_BYTES = NW * 16 * 16 * 4;  // per wave: its 16 x 16 diagonal block of L (fp32)
  constexpr int LDS = (XLO ? 2 : 1) * KN_BYTES + (LO ? 2 : 1) * VT_BYTES + SB_BYTES + SL_BYTES + BC_BYTES + WT_BYTES + BT_BYTES +
                      LB_BYTES;
  constexpr int NS = NDT * NDT;
  constexpr int TPW = (NS + NW - 1) / NW;
  static_assert(NTOK >= 1 && NQ >= 1 && CB <= 64 && 64 % CB == 0 && RH * P == NDT, "unsupported head size");
  static_assert(ESZ == 4 || NTOK % 2 == 0, "bf16 V^T writes pack token pairs");
  static_assert(32 % TW == 0 && LOADERS % 64 == 0, "whole loader waves cover tokens 0..31");
  static_assert(LDS <= 160 * 1024, "LDS budget");

  constexpr int RHP = recur_heads<D, NTH, G>(LDS);  // heads per pass of the token-by-token re-evaluation
  // the rescaled-key forms (not RAW) with a decay can meet decays too strong for them
  constexpr bool RERUN = !RAW && DK != 0;
  static_assert(!RERUN || RHP >= 1, "LDS for the token-by-token re-evaluation");
  __shared__ __align__(16) unsigned char smem[LDS + 16];
  __shared__ int rerun_flag;  // some chunk's decays exceed kDeltaExactSpan
  unsigned char* sp = smem;
  auto carve = [&](int bytes) {
    unsigned char* p = sp;
    sp += bytes;
    return p;
  };
  DT* Kh = (DT*)carve(KN_BYTES);                  // k^ = k e^{c_sigma - b} (hi)
  DT* Kl = (DT*)carve(XLO ? KN_BYTES : 0);        // its lo part
  DT* Vt = (DT*)carve(VT_BYTES);                  // V^T, then U^T (hi)
  DT* Vl = (DT*)carve(LO ? VT_BYTES : 0);         // lo parts
  DT* Sb = (DT*)carve(SB_BYTES);                  // S^T of the state before the chunk
  DT* Sl = (DT*)carve(SL_BYTES);                  // its lo part (SLO)
  float* Bc = (float*)carve(BC_BYTES);            // b_t per key dim (DK == 2)
  float* Wt = (float*)carve(WT_BYTES);            // loader-wave totals of the scan
  float* Bt = (float*)carve(BT_BYTES);            // beta_t, then (per-head decay) b_t
  float* Lb = (float*)carve(LB_BYTES);            // per wave: L of its diagonal block

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the two waves of a row block sit on different SIMDs (w % 4)
  const int hp = P == 2 ? (w & 1) : 0, wr = P == 2 ? (w >> 1) : w;
  int l = tid & 63, lr = l & 15, lg = l >> 4;
  // query-head group hg of hs (the group's heads are G of the kv head's G * hs)
  // and segment s of ns: tokens [t0, t0 + T) of the unit's sequence
  const int hs = a.hsplit > 1 ? a.hsplit : 1;
  const int ns = a.nseg > 1 ? a.nseg : 1;
  const int hc = a.hg_count > 0 ? a.hg_count : hs;  // groups of this launch, from hg_first
  const int hg = a.hg_first + blockIdx.x % hc;
  const int us = blockIdx.x / hc;
  const int u = us / ns, s = us % ns;
  const int Hq = a.Hq, Hkv = a.Hkv, TT = a.T;
  const int sl = a.seg_len > 0 ? a.seg_len : TT;  // (a single segment may be shorter than the sequence)
  const int t0 = s * sl;
  const int T = min(TT, t0 + sl) - t0;
  const int b = u / Hkv, j = u % Hkv;
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int QS = Hq * D, KS = Hkv * D;
  const int64_t row0 = (int64_t)b * TT + t0;  // the segment's first row
  const IT* qb = (const IT*)a.q + row0 * QS + (int64_t)(j * G * hs + hg * G) * D;
  IT* ob = a.out ? (IT*)a.out + row0 * QS + (int64_t)(j * G * hs + hg * G) * D : nullptr;
  const IT* kb = (const IT*)a.k + row0 * KS + (int64_t)j * D;
  const IT* vb = a.v ? (const IT*)a.v + row0 * KS + (int64_t)j * D : nullptr;
  const IT* gb = DK == 2 ? (const IT*)a.decay + row0 * KS + (int64_t)j * D
                         : (DK == 1 ? (const IT*)a.decay + row0 * Hkv + j : nullptr);
  const IT* betab = (const IT*)a.beta + row0 * a.beta_heads + (a.beta_heads > 1 ? j : 0);
  const float* s_in = a.s_in ? a.s_in + u * a.s_in_u + s * a.s_in_s : nullptr;
  float* s_out = (a.s_out && hg == 0 && (a.s_out_all || s == ns - 1)) ? a.s_out + u * a.s_out_u + s * a.s_out_s
                                                                      : nullptr;
  const float scale = a.scale;
  auto vt_at = [&](int r, int blk) { return r * VT_LD + ((blk ^ vt_swz(r)) * VEC); };
  auto kn_at = [&](int t, int col) {
    const int sw = SWZ ? ksw<CB>(t) : (kn_swz(t) & (CB - 1));
    return t * KN_LD + ((((col / VEC) ^ sw) & (CB - 1)) * VEC) + (col % VEC);
  };
  auto sq_at = [&](int r, int col) {
    const int sw = SWZ ? qsw<CB>(r) : sq_swz(r);
    return r * SB_LD + ((((col / VEC) ^ sw) & (CB - 1)) * VEC) + (col % VEC);
  };
  auto to_f = [&](DT x) -> float {
    if constexpr (ESZ == 2) return bf16_bits_to_f32(x);
    else return x;
  };
  // fp32 value -> operand hi (and lo) words, for pairs packed the way O::pack does
  auto split8 = [&](const float (&f)[VEC], u32x4_t& hi, u32x4_t& lo) {
    hi = O::pack(f);
    if constexpr (LO) {
      float r[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) r[e] = f[e] - bf16_bits_to_f32((hi[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      lo = O::pack(r);
    }
  };

  // four fp32 values -> bf16 hi + lo operands of a 16x16x16 MFMA
  auto split4 = [&](const float (&f)[4], s16x4_t& hi, s16x4_t& lo) {
    u32x2_t h, r;
    h[0] = pack_bf16x2(f[0], f[1]);
    h[1] = pack_bf16x2(f[2], f[3]);
    r[0] = pack_bf16x2(f[0] - __uint_as_float(h[0] << 16), f[1] - __uint_as_float(h[0] & 0xffff0000u));
    r[1] = pack_bf16x2(f[2] - __uint_as_float(h[1] << 16), f[3] - __uint_as_float(h[1] & 0xffff0000u));
    hi = __builtin_bit_cast(s16x4_t, h);
    lo = __builtin_bit_cast(s16x4_t, r);
  };

  // ---- state tiles: wave w owns tiles tau = w*TPW + i (rows rt, columns ct)
  f32x4_t sacc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) sacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (s_in) {
    const float* sin = s_in;
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
  auto write_sb = [&]() {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tau = w * TPW + i;
      if (tau < NS) {
        const int rt = tau / NDT, ct = tau % NDT;
        const int off = sq_at(16 * ct + lr, 16 * rt + 4 * lg);
        DT* p = Sb + off;
        if constexpr (ESZ == 2) {
          u32x2_t v2;
          v2[0] = pack_bf16x2(sacc[i][0], sacc[i][1]);
          v2[1] = pack_bf16x2(sacc[i][2], sacc[i][3]);
          *(u32x2_t*)p = v2;
          if constexpr (SLO) {
            u32x2_t l2;
            l2[0] = pack_bf16x2(sacc[i][0] - __uint_as_float(v2[0] << 16), sacc[i][1] - __uint_as_float(v2[0] & 0xffff0000u));
            l2[1] = pack_bf16x2(sacc[i][2] - __uint_as_float(v2[1] << 16), sacc[i][3] - __uint_as_float(v2[1] & 0xffff0000u));
            *(u32x2_t*)(Sl + off) = l2;
          }
        } else {
          *(f32x4_t*)p = sacc[i];
        }
      }
    }
  };
  write_sb();

  const int cb = tid % CB, tg = tid / CB;
  const bool loader = tid < LOADERS;
  u32x4_t pk[NTOK], pv[NTOK], pg[DK == 2 ? NTOK : 1];

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


  // a scalar of the I/O type (beta, a per-head decay) as fp32
  auto ld1 = [&](const IT* p) -> float {
    if constexpr (sizeof(IT) == 2) return Io<IT>::to_f32(*(const uint16_t*)p);
    else return *(const float*)p;
  };

  int tq = 16 * wr + lr;
  // The lane indices pass through an empty asm at the start of every phase, so
  // that the swizzled LDS addresses derived from them are formed inside the
  // phase instead of being hoisted out of the chunk loop and held (or spilled)
  // across all of it.
  auto refresh = [&]() {
    int x = tid & 63;
    asm volatile("" : "+v"(x));
    l = x;
    lr = x & 15;
    lg = x >> 4;
    tq = 16 * wr + lr;
  };
  // ---- prefetch: a chunk's k, v (and per-dim decays) into the loaders'
  // registers, beta and the per-head decay of token l into wave 0's.  The
  // addresses are clamped to the last token, so the loop's prefetch of the
  // chunk after the last reloads the last; tokens past the end are zeroed when
  // staged.
  float pbe = 0.f, pgx = 0.f;
  auto prefetch = [&](int c) {
    const int tb = c * kChunk;
    if (w == 0) {
      const int tc = min(tb + l, T - 1);
      pbe = ld1(betab + (int64_t)tc * a.beta_heads);
      if constexpr (DK == 1) pgx = ld1(gb + (int64_t)tc * Hkv);
    }
    if (loader) {
#pragma unroll
      for (int n = 0; n < NTOK; ++n) {
        const int64_t off = (int64_t)min(tb + tg * NTOK + n, T - 1) * KS + cb * VEC;
        pk[n] = ld16(kb + off);
        pv[n] = vb ? ld16(vb + off) : u32x4_t{0u, 0u, 0u, 0u};
        if constexpr (DK == 2) pg[n] = ld16(gb + off);
      }
    }
  };

  // ---- stage: beta and b_t (per-head decays: wave 0's scan), V^T (hi + lo),
  // b_t -> Bc, k^ = k e^{c_sigma - b} (hi + lo) -> Kh, Kl.  Two barriers.  The
  // lane's own key row for the solve is loaded first, to arrive meanwhile.
  u32x4_t kr[NQ];
  auto stage = [&](int c) {
    const int tb = c * kChunk;
    {
      const int tokc = min(tb + tq, T - 1);
#pragma unroll
      for (int m = 0; m < NQ; ++m) kr[m] = ld16(kb + (int64_t)tokc * KS + KB * m + VEC * lg);
    }
    if (w == 0) {
      const bool ok = tb + l < T;
      Bt[l] = ok ? pbe : 0.f;  // tokens past the end: beta = 0, so u = 0
      if constexpr (DK == 1) {
        float x = ok ? pgx : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off);
          if (l >= off) x += y;
        }
        Bt[kChunk + l] = x;
      }
    }
    float bx[NTOK][VEC];
    float tot[VEC];
    if (loader) {
#pragma unroll
      for (int n = 0; n < NTOK; ++n) {
        if (tb + tg * NTOK + n >= T) {
          pk[n] = u32x4_t{0u, 0u, 0u, 0u};
          pv[n] = u32x4_t{0u, 0u, 0u, 0u};
          if constexpr (DK == 2) pg[n] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
      if constexpr (LO) {
        u32x4_t pl[NTOK];
#pragma unroll
        for (int n = 0; n < NTOK; ++n) {
          float f[VEC];
          Io<IT>::unpack(pv[n], f);
          split8(f, pv[n], pl[n]);
        }
        write_vt(Vl, pl);
      }
      write_vt(Vt, pv);
      if constexpr (DK == 2) {
#pragma unroll
        for (int n = 0; n < NTOK; ++n) Io<IT>::unpack(pg[n], bx[n]);
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
          tot[e] = x - own;
          if (l >= 64 - CB) Wt[w * D + cb * VEC + e] = x;
        }
      }
    }
    __syncthreads();
    if (loader) {
      float c32[VEC];
      if constexpr (DK == 2) {
        float off[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          off[e] = tot[e];
          c32[e] = 0.f;
        }
        for (int w2 = 0; w2 < w; ++w2) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) off[e] += Wt[w2 * D + cb * VEC + e];
        }
        constexpr int W32 = 32 / TW;
#pragma unroll
        for (int w2 = 0; w2 < W32; ++w2)
#pragma unroll
          for (int e = 0; e < VEC; ++e) c32[e] += Wt[w2 * D + cb * VEC + e];
#pragma unroll
        for (int n = 0; n < NTOK; ++n)
#pragma unroll
          for (int e = 0; e < VEC; ++e) bx[n][e] += off[e];
      } else {
#pragma unroll
        for (int n = 0; n < NTOK; ++n) {
          const float bt = DK == 1 ? Bt[kChunk + tg * NTOK + n] : 0.f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) bx[n][e] = bt;
        }
        const float c31 = DK == 1 ? Bt[kChunk + 31] : 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) c32[e] = c31;
      }
      if constexpr (RERUN) {
        float span = 0.f;
#pragma unroll
        for (int n = 0; n < NTOK; ++n)
#pragma unroll
          for (int e = 0; e < VEC; ++e) span = fmaxf(span, fabsf(bx[n][e]));
        if (!(span <= kDeltaExactSpan)) rerun_flag = 1;  // (NaN decays too)
      }
#pragma unroll
      for (int n = 0; n < NTOK; ++n) {
        const int t = tg * NTOK + n;
        if constexpr (DK == 2) {
#pragma unroll
          for (int e = 0; e < VEC; e += 4)
            *(f32x4_t*)(Bc + t * BC_LD + cb * VEC + e) = f32x4_t{bx[n][e], bx[n][e + 1], bx[n][e + 2], bx[n][e + 3]};
        }
        float kx[VEC], kh[VEC];
        Io<IT>::unpack(pk[n], kx);
#pragma unroll
        for (int e = 0; e < VEC; ++e) kh[e] = RAW ? kx[e] : kx[e] * __expf((t >= 32 ? c32[e] : 0.f) - bx[n][e]);
        u32x4_t hi, lo;
        split8(kh, hi, lo);
        st16(Kh + kn_at(t, cb * VEC), hi);
        if constexpr (XLO) st16(Kl + kn_at(t, cb * VEC), lo);
      }
    }
    __syncthreads();
  };

  // Row tq's vector x (operand layout, raw I/O words), times e^{b_tq - c} with
  // c = 0 (second == false) or b_31, split into hi (+ lo) operands.  The row
  // offsets pass through an empty asm so that each use recomputes the factors
  // instead of the compiler keeping them live across heads.
  auto scaled = [&](const u32x4_t (&x)[NQ], u32x4_t (&hi)[NQ], u32x4_t (&lo)[LO ? NQ : 1], bool second) {
    if constexpr (RAW) {
#pragma unroll
      for (int m = 0; m < NQ; ++m) hi[m] = x[m];
      return;
    }
    int rt_off = tq * BC_LD, r31_off = 31 * BC_LD;
    asm volatile("" : "+v"(rt_off), "+v"(r31_off));
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
      const int d0 = KB * m + VEC * lg;
      float f[VEC];
      Io<IT>::unpack(x[m], f);
      if constexpr (DK == 2) {
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const f32x4_t bt = *(const f32x4_t*)(Bc + rt_off + d0 + e);
          f32x4_t cs = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (second) cs = *(const f32x4_t*)(Bc + r31_off + d0 + e);
#pragma unroll
          for (int i = 0; i < 4; ++i) f[e + i] *= __expf(bt[i] - cs[i]);
        }
      } else if constexpr (DK == 1) {
        const float fac = __expf(Bt[kChunk + tq] - (second ? Bt[kChunk + 31] : 0.f));
#pragma unroll
        for (int e = 0; e < VEC; ++e) f[e] *= fac;
      }
      u32x4_t h, lw;
      split8(f, h, lw);
      hi[m] = h;
      if constexpr (XLO) lo[m] = lw;
    }
  };
  // key row of A^T / L^T tile t (bf16: tile pairs over 32 keys with permuted
  // rows, element q of tile t at key key_of(t, q); fp32: 16-key tiles)
  auto key_of = [&](int t, int q) {
    return ESZ == 2 ? 32 * (t >> 1) + 8 * lg + 4 * (t & 1) + q : 16 * t + 4 * lg + q;
  };
  // RAW with a per-head decay: element q of tile t times exp(b_row - b_key),
  // selected to 0 where key > row (or key >= row when strict), never
  // multiplied there (the factor may overflow past the diagonal)
  auto decay_tile = [&](f32x4_t at, int t, int row, bool strict) {
    const float br = Bt[kChunk + row];
    const f32x4_t bk = *(const f32x4_t*)(Bt + kChunk + key_of(t, 0));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int key = key_of(t, q);
      at[q] = (strict ? key < row : key <= row) ? at[q] * __expf(br - bk[q]) : 0.f;
    }
    return at;
  };
  // unmasked tile t of (k^ rows) x (the lane's scaled row): Kh xh + Kl xh + Kh xl
  auto k_tile = [&](int t, const u32x4_t (&xh)[NQ], const u32x4_t (&xl)[LO ? NQ : 1]) {
    f32x4_t at = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int krow = ESZ == 2 ? 32 * (t >> 1) + 8 * (lr >> 2) + 4 * (t & 1) + (lr & 3) : 16 * t + lr;
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
      const u32x4_t kh = ld16(Kh + kn_at(krow, KB * m + VEC * lg));
      O::mma(at, kh, xh[m]);
      if constexpr (XLO) {
        O::mma(at, ld16(Kl + kn_at(krow, KB * m + VEC * lg)), xh[m]);
        O::mma(at, kh, xl[m]);
      }
    }
    return at;
  };
  // bf16 hi + lo B operands of a tile pair (keys of pair p along the contraction)
  auto pair_operands = [&](const f32x4_t& at0, const f32x4_t& at1, u32x4_t& bh, u32x4_t& bl) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x4_t& at = (e >> 1) ? at1 : at0;
      const float x0 = at[2 * (e & 1)], x1 = at[2 * (e & 1) + 1];
      const uint32_t hw = pack_bf16x2(x0, x1);
      bh[e] = hw;
      bl[e] = pack_bf16x2(x0 - __uint_as_float(hw << 16), x1 - __uint_as_float(hw & 0xffff0000u));
    }
  };

  // ---- query rows of head part hp, head hh, in two register sets that
  // alternate between heads: each head's rows are requested one step ahead
  // (the first during the solve), and no register still being loaded is copied
  u32x4_t qbuf[2][NQ];
  auto load_q = [&](int c, int hh) {
    const int tokc = min(c * kChunk + tq, T - 1);
    const int hq = hp + P * hh;
#pragma unroll
    for (int m = 0; m < NQ; ++m) qbuf[hh & 1][m] = ld16(qb + (int64_t)tokc * QS + hq * D + KB * m + VEC * lg);
  };

  // ---- pseudo-values.  Wave (hp, wr) owns rows [16wr, 16wr+16) of the chunk
  // and dv tiles hp*RH .. hp*RH + RH - 1, held token-major: lane (lg, lr) holds
  // rows 16wr + 4lg + q of value dim 16ct + lr, which is also the B operand
  // layout of a 16x16x16 MFMA over those rows.
  //   1. R = beta (V - Kbar S_0) for its rows;
  //   2. its rows of L: the strictly lower diagonal block -> LDS, the part left
  //      of it -> MFMA operands (hi + lo);
  //   3. T = (I + diag(beta) L_ii)^-1 of its diagonal block: row lr of T in
  //      every lane group, by back substitution in registers (no lane traffic);
  //   4. block by block, a barrier after each: X = R - beta sum_{j<i} L_ij U_j
  //      over the U rows already written, then U_i = T X by MFMA, stored as
  //      U^T over the consumed V^T columns.
  auto solve = [&](int c) {
    refresh();
    u32x4_t k0h[NQ], k0l[LO ? NQ : 1];
    scaled(kr, k0h, k0l, false);  // kbar, also the first key block's scaled row
    const int r0 = 16 * wr + 4 * lg;  // the lane's first row
    const f32x4_t bet4 = *(const f32x4_t*)(Bt + r0);
    // element offset of the lane's 4 rows in row `row` of V^T / U^T
    auto row4_at = [&](int row) { return vt_at(row, r0 / VEC) + r0 % VEC; };
    f32x4_t val[RH];
#pragma unroll
    for (int i = 0; i < RH; ++i) val[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
#pragma unroll
      for (int i = 0; i < RH; ++i) {
        const int so = sq_at(16 * (hp * RH + i) + lr, KB * m + VEC * lg);
        const u32x4_t av = ld16(Sb + so);
        O::mma(val[i], k0h[m], av);
        if constexpr (XLO) O::mma(val[i], k0l[m], av);
        if constexpr (SLO) O::mma(val[i], k0h[m], ld16(Sl + so));
      }
    }
#pragma unroll
    for (int i = 0; i < RH; ++i) {
      const int off = row4_at(16 * (hp * RH + i) + lr);
      float v[4];
      if constexpr (ESZ == 2) {
        const u32x2_t h2 = *(const u32x2_t*)(Vt + off);
        v[0] = __uint_as_float(h2[0] << 16);
        v[1] = __uint_as_float(h2[0] & 0xffff0000u);
        v[2] = __uint_as_float(h2[1] << 16);
        v[3] = __uint_as_float(h2[1] & 0xffff0000u);
        if constexpr (LO) {
          const u32x2_t l2 = *(const u32x2_t*)(Vl + off);
          v[0] += __uint_as_float(l2[0] << 16);
          v[1] += __uint_as_float(l2[0] & 0xffff0000u);
          v[2] += __uint_as_float(l2[1] << 16);
          v[3] += __uint_as_float(l2[1] & 0xffff0000u);
        }
      } else {
        const f32x4_t v4 = *(const f32x4_t*)(Vt + off);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = v4[q];
      }
      if constexpr (RAWDEC) {
        // Kbar S_0 from the raw keys: row t times exp(b_t)
        const f32x4_t b4 = *(const f32x4_t*)(Bt + kChunk + r0);
#pragma unroll
        for (int q = 0; q < 4; ++q) val[i][q] *= __expf(b4[q]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) val[i][q] = bet4[q] * (v[q] - val[i][q]);
    }

    // L over the wave's rows.  bf16: key pairs p <= wr/2 (off-diagonal
    // operands oh/ol, keys >= 16wr zeroed); fp32: 16-key tiles t < wr (ot).
    float* lb = Lb + w * 256;
    u32x4_t oh[ESZ == 2 ? 2 : 1], ol[ESZ == 2 ? 2 : 1];
    f32x4_t ot[ESZ == 4 ? 3 : 1];
    {
      u32x4_t k1h[NQ], k1l[LO ? NQ : 1];
      if (wr >= 2) scaled(kr, k1h, k1l, true);
      if constexpr (ESZ == 2) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          if (32 * p <= 16 * wr + 15) {
            f32x4_t at0 = p == 0 ? k_tile(0, k0h, k0l) : k_tile(2, k1h, k1l);
            f32x4_t at1 = p == 0 ? k_tile(1, k0h, k0l) : k_tile(3, k1h, k1l);
            if constexpr (RAWDEC) {
              at0 = decay_tile(at0, 2 * p, tq, true);
              at1 = decay_tile(at1, 2 * p + 1, tq, true);
            }
            // the diagonal block's keys 16wr + 8(lg & 1) + 4odd + q sit in
            // lane groups 2(wr & 1) and 2(wr & 1) + 1 of pair wr / 2
            if (p == (wr >> 1) && (lg >> 1) == (wr & 1)) {
#pragma unroll
              for (int odd = 0; odd < 2; ++odd) {
                f32x4_t x = odd ? at1 : at0;
#pragma unroll
                for (int q = 0; q < 4; ++q) x[q] = 8 * (lg & 1) + 4 * odd + q < lr ? x[q] : 0.f;
                *(f32x4_t*)(lb + lr * 16 + 8 * (lg & 1) + 4 * odd) = x;
              }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              at0[q] = key_of(2 * p, q) < 16 * wr ? at0[q] : 0.f;
              at1[q] = key_of(2 * p + 1, q) < 16 * wr ? at1[q] : 0.f;
            }
            pair_operands(at0, at1, oh[p], ol[p]);
          }
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t <= wr) {
            f32x4_t at = t < 2 ? k_tile(t, k0h, k0l) : k_tile(t, k1h, k1l);
            if constexpr (RAWDEC) at = decay_tile(at, t, tq, true);
            if (t == wr) {
              f32x4_t x = at;
#pragma unroll
              for (int q = 0; q < 4; ++q) x[q] = 4 * lg + q < lr ? x[q] : 0.f;
              *(f32x4_t*)(lb + lr * 16 + 4 * lg) = x;
            } else if (t < 3) {
              ot[t] = at;
            }
          }
        }
      }
    }
    // row lr of T, columns 4lg .. 4lg+3 in lane group lg: y (I + diag(beta) L_ii)
    // = e_lr, solved by 4-column blocks from the last.  Block s is finished by
    // group s from the sums gathered so far, then sent to the lower groups,
    // which add its terms to their sums (the other groups' sums are not used
    // again and take the same arithmetic unmasked).
    float t4[4] = {0.f, 0.f, 0.f, 0.f}, acc4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sb = 3; sb >= 0; --sb) {
      f32x4_t lrow[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) lrow[e] = *(const f32x4_t*)(lb + 16 * (4 * sb + e) + 4 * lg);
      const f32x4_t bs = *(const f32x4_t*)(Bt + 16 * wr + 4 * sb);
      float z[4];
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        float v = (lr == 4 * sb + e ? 1.f : 0.f) - acc4[e];
#pragma unroll
        for (int e2 = e + 1; e2 < 4; ++e2) v -= bs[e2] * lrow[e2][e] * z[e2];
        z[e] = v;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) t4[e] = lg == sb ? z[e] : t4[e];
      if (sb > 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float by = bs[e] * __shfl(t4[e], 16 * sb + lr);
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) acc4[e2] += lrow[e][e2] * by;
        }
      }
    }
    s16x4_t th, tl;
    if constexpr (ESZ == 2) split4(t4, th, tl);

    if (ob) {
      load_q(c, 0);
      if constexpr (PAIR) load_q(c, 1);
    }
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      if (wr == blk) {
        if (blk > 0) {
          f32x4_t cacc[RH];
#pragma unroll
          for (int i = 0; i < RH; ++i) cacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < RH; ++i) {
            const int row = 16 * (hp * RH + i) + lr;
            if constexpr (ESZ == 2) {
#pragma unroll
              for (int p = 0; p < 2; ++p) {
                if (32 * p < 16 * blk) {
                  const u32x4_t uh = ld16(Vt + vt_at(row, 4 * p + lg));
                  O::mma(cacc[i], oh[p], uh);
                  O::mma(cacc[i], ol[p], uh);
                  O::mma(cacc[i], oh[p], ld16(Vl + vt_at(row, 4 * p + lg)));
                }
              }
            } else {
#pragma unroll
              for (int t = 0; t < 3; ++t) {
                if (t < blk) {
                  const u32x4_t uv = ld16(Vt + vt_at(row, 4 * t + lg));
#pragma unroll
                  for (int q = 0; q < 4; ++q)
                    cacc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(ot[t][q], __uint_as_float(uv[q]), cacc[i], 0, 0, 0);
                }
              }
            }
          }
#pragma unroll
          for (int i = 0; i < RH; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) val[i][q] -= bet4[q] * cacc[i][q];
        }
#pragma unroll
        for (int i = 0; i < RH; ++i) {
          f32x4_t uo = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if constexpr (ESZ == 2) {
            s16x4_t xh, xl;
            const float x4[4] = {val[i][0], val[i][1], val[i][2], val[i][3]};
            split4(x4, xh, xl);
            uo = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(th, xh, uo, 0, 0, 0);
            uo = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(tl, xh, uo, 0, 0, 0);
            uo = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(th, xl, uo, 0, 0, 0);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) uo = __builtin_amdgcn_mfma_f32_16x16x4f32(t4[q], val[i][q], uo, 0, 0, 0);
          }
          const int off = row4_at(16 * (hp * RH + i) + lr);
          if constexpr (ESZ == 2) {
            u32x2_t h2, l2;
            h2[0] = pack_bf16x2(uo[0], uo[1]);
            h2[1] = pack_bf16x2(uo[2], uo[3]);
            l2[0] = pack_bf16x2(uo[0] - __uint_as_float(h2[0] << 16), uo[1] - __uint_as_float(h2[0] & 0xffff0000u));
            l2[1] = pack_bf16x2(uo[2] - __uint_as_float(h2[1] << 16), uo[3] - __uint_as_float(h2[1] & 0xffff0000u));
            *(u32x2_t*)(Vt + off) = h2;
            *(u32x2_t*)(Vl + off) = l2;
          } else {
            *(f32x4_t*)(Vt + off) = uo;
          }
        }
      }
      __syncthreads();
    }
  };

  // ---- outputs of the chunk's queries (per head), with U in V's place
  auto outputs = [&](int c) {
    const int tok = c * kChunk + tq;
    auto need = [&](int t) { return ESZ == 2 ? (32 * (t >> 1) <= 16 * wr + 15) : (t <= wr); };
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      refresh();
      const int hq = hp + P * hh;
      if (hh + 1 < HPW) load_q(c, hh + 1);
      const u32x4_t (&qr)[NQ] = qbuf[hh & 1];
      u32x4_t qop[NQ], qlo[LO ? NQ : 1];
      scaled(qr, qop, qlo, false);
      auto a_tile = [&](int t) {
        f32x4_t at = k_tile(t, qop, qlo);
        if constexpr (RAWDEC) return decay_tile(at, t, tq, false);
#pragma unroll
        for (int q = 0; q < 4; ++q) at[q] = key_of(t, q) <= tq ? at[q] : 0.f;
        return at;
      };
      f32x4_t a0[2];
      a0[0] = a_tile(0);
      a0[1] = need(1) ? a_tile(1) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      f32x4_t nacc[NDT];
#pragma unroll
      for (int ct = 0; ct < NDT; ++ct) nacc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < NQ; ++m) {
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) {
          const int so = sq_at(16 * ct + lr, KB * m + VEC * lg);
          const u32x4_t av = ld16(Sb + so);
          O::mma(nacc[ct], av, qop[m]);
          if constexpr (XLO) O::mma(nacc[ct], av, qlo[m]);
          if constexpr (SLO) O::mma(nacc[ct], ld16(Sl + so), qop[m]);
        }
      }
      if constexpr (RAWDEC) {
        // q S_0 from the raw query: times exp(b_t) of the lane's token
        const float eb = __expf(Bt[kChunk + tq]);
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) nacc[ct] *= eb;
      }
      if constexpr (ESZ == 2) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          if (need(2 * p)) {
            f32x4_t at0 = a0[0], at1 = a0[1];
            if (p == 1) {
              if constexpr (!RAW) scaled(qr, qop, qlo, true);
              at0 = a_tile(2);
              at1 = a_tile(3);
            }
            u32x4_t bh, bl;
            pair_operands(at0, at1, bh, bl);
#pragma unroll
            for (int ct = 0; ct < NDT; ++ct) {
              const u32x4_t uh = ld16(Vt + vt_at(16 * ct + lr, 4 * p + lg));
              O::mma(nacc[ct], uh, bh);
              O::mma(nacc[ct], uh, bl);
              O::mma(nacc[ct], ld16(Vl + vt_at(16 * ct + lr, 4 * p + lg)), bh);
            }
          }
        }
      } else {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          if (need(jt)) {
            if (!RAW && jt == 2) scaled(qr, qop, qlo, true);
            const f32x4_t at = jt < 2 ? a0[jt] : a_tile(jt);
#pragma unroll
            for (int ct = 0; ct < NDT; ++ct) {
              const u32x4_t uv = ld16(Vt + vt_at(16 * ct + lr, 4 * jt + lg));
#pragma unroll
              for (int q = 0; q < 4; ++q)
                nacc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(uv[q]), at[q], nacc[ct], 0, 0, 0);
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
  };

  // ---- the same for RAW bf16 inputs with an even number of heads per wave:
  // the heads go in pairs, and each S^T (hi, lo) and U^T (hi, lo) operand is
  // read from LDS once for both heads of a pair
  auto outputs_pair = [&](int c) {
    const int tok = c * kChunk + tq;
    auto need = [&](int t) { return 32 * (t >> 1) <= 16 * wr + 15; };
#pragma unroll
    for (int hh = 0; hh < HPW; hh += 2) {
      refresh();
      if (hh > 0) {
        load_q(c, hh);
        load_q(c, hh + 1);
      }
      const u32x4_t (&qa)[NQ] = qbuf[0];
      const u32x4_t (&qb2)[NQ] = qbuf[1];
      u32x4_t unused[LO ? NQ : 1];  // lo operands: never read on the RAW path
      f32x4_t n0[NDT], n1[NDT];
#pragma unroll
      for (int ct = 0; ct < NDT; ++ct) {
        n0[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        n1[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int m = 0; m < NQ; ++m) {
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) {
          const int so = sq_at(16 * ct + lr, KB * m + VEC * lg);
          const u32x4_t av = ld16(Sb + so);
          const u32x4_t al = ld16(Sl + so);
          O::mma(n0[ct], av, qa[m]);
          O::mma(n1[ct], av, qb2[m]);
          O::mma(n0[ct], al, qa[m]);
          O::mma(n1[ct], al, qb2[m]);
        }
      }
      if constexpr (RAWDEC) {
        const float eb = __expf(Bt[kChunk + tq]);
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) {
          n0[ct] *= eb;
          n1[ct] *= eb;
        }
      }
      auto a_tile = [&](int t, const u32x4_t (&x)[NQ]) {
        f32x4_t at = k_tile(t, x, unused);
        if constexpr (RAWDEC) return decay_tile(at, t, tq, false);
#pragma unroll
        for (int q = 0; q < 4; ++q) at[q] = key_of(t, q) <= tq ? at[q] : 0.f;
        return at;
      };
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (need(2 * p)) {
          u32x4_t bh0, bl0, bh1, bl1;
          pair_operands(a_tile(2 * p, qa), a_tile(2 * p + 1, qa), bh0, bl0);
          pair_operands(a_tile(2 * p, qb2), a_tile(2 * p + 1, qb2), bh1, bl1);
#pragma unroll
          for (int ct = 0; ct < NDT; ++ct) {
            const u32x4_t uh = ld16(Vt + vt_at(16 * ct + lr, 4 * p + lg));
            const u32x4_t ul = ld16(Vl + vt_at(16 * ct + lr, 4 * p + lg));
            O::mma(n0[ct], uh, bh0);
            O::mma(n1[ct], uh, bh1);
            O::mma(n0[ct], uh, bl0);
            O::mma(n1[ct], uh, bl1);
            O::mma(n0[ct], ul, bh0);
            O::mma(n1[ct], ul, bh1);
          }
        }
      }
      if (tok < T) {
        IT* orow0 = ob + (int64_t)tok * QS + (hp + P * hh) * D + 4 * lg;
        IT* orow1 = ob + (int64_t)tok * QS + (hp + P * (hh + 1)) * D + 4 * lg;
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) {
          store4(orow0 + 16 * ct, scale * n0[ct][0], scale * n0[ct][1], scale * n0[ct][2], scale * n0[ct][3]);
          store4(orow1 + 16 * ct, scale * n1[ct][0], scale * n1[ct][1], scale * n1[ct][2], scale * n1[ct][3]);
        }
      }
    }
  };

  // ---- state: S = diag(e^{b_C}) S + sum_j diag(e^{b_C - b_j}) k_j u_j^T, the
  // decayed keys from k^ (hi + lo) times e^{b_C - c_sigma} in fp32, then hi + lo
  int cl = kChunk - 1;  // the chunk's last token (the sequence's last in a partial chunk)
  auto update = [&]() {
    refresh();
    u32x4_t kop[NKS], kol[NKS];
    float er[4];  // per-dim decay of state rows 16 rt + 4 lg + q over the chunk (shared by a row tile's column tiles)
    int cur_rt = -1;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tau = w * TPW + i;
      if (tau < NS) {
        const int rt = tau / NDT, ct = tau % NDT;
        if constexpr (DK == 1) sacc[i] *= __expf(Bt[kChunk + cl]);
        if (rt != cur_rt) {
          cur_rt = rt;
          if constexpr (DK == 2) {
#pragma unroll
            for (int q = 0; q < 4; ++q) er[q] = __expf(Bc[cl * BC_LD + 16 * rt + 4 * lg + q]);
          }
          const int dk = 16 * rt + lr;
          const float bC = DK == 2 ? Bc[cl * BC_LD + dk] : (DK == 1 ? Bt[kChunk + cl] : 0.f);
          const float c31 = DK == 2 ? Bc[31 * BC_LD + dk] : (DK == 1 ? Bt[kChunk + 31] : 0.f);
#pragma unroll
          for (int m = 0; m < NKS; ++m) {
            float f[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              const int sk = KB * m + VEC * lg + e;
              const int off = kn_at(sk, dk);
              float kv = to_f(Kh[off]);
              if constexpr (XLO) kv += to_f(Kl[off]);
              f[e] = DK == 0 ? kv : kv * __expf(bC - (RAW ? Bt[kChunk + sk] : (sk >= 32 ? c31 : 0.f)));
            }
            split8(f, kop[m], kol[m]);
          }
        }
        if constexpr (DK == 2) {
#pragma unroll
          for (int q = 0; q < 4; ++q) sacc[i][q] *= er[q];
        }
#pragma unroll
        for (int m = 0; m < NKS; ++m) {
          const u32x4_t uh = ld16(Vt + vt_at(16 * ct + lr, (KB / VEC) * m + lg));
          O::mma(sacc[i], kop[m], uh);
          if constexpr (LO) {
            O::mma(sacc[i], kol[m], uh);
            O::mma(sacc[i], kop[m], ld16(Vl + vt_at(16 * ct + lr, (KB / VEC) * m + lg)));
          }
        }
      }
    }
  };

  prefetch(0);
  if (tid == 0) rerun_flag = 0;  // (read only after the chunk loop's barriers)
  for (int c = 0; c < nchunks; ++c) {
    // (its cumulative decay is then exactly the newest token's, whatever order
    // the scan summed the padded zeros in)
    cl = min(kChunk, T - c * kChunk) - 1;
    stage(c);
    prefetch(min(c + 1, nchunks - 1));
    solve(c);
    if (ob) {
      if constexpr (PAIR)
        outputs_pair(c);
      else
        outputs(c);
    }
    update();
    __syncthreads();
    write_sb();
  }
  // (with a re-evaluation below the state is stored by it: stored here, it
  // would overwrite a start state the re-evaluation reads when the state is
  // updated in place)
  if (s_out && !(RERUN && rerun_flag)) {
    float* sout = s_out;
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
  if constexpr (RERUN) {
    __syncthreads();  // the chunk loop and any state stores above are done
    if (rerun_flag) {
      // strong decays: the whole sequence again, token by token, outputs and state
      RecurPtrs rp;
      rp.q = qb;
      rp.k = kb;
      rp.v = vb;
      rp.decay = gb;
      rp.beta = betab;
      rp.out = ob;
      rp.s_in = s_in;
      rp.s_out = s_out;
      rp.qs = QS;
      rp.ks = KS;
      rp.gs = DK == 2 ? KS : Hkv;
      rp.bs = a.beta_heads;
      rp.t0 = 0;
      rp.t1 = T;
      rp.scale = scale;
      token_recurrence<IT, D, NTH, G, RHP, DK, true>(smem, rp);
    }
  }
}

// FULL: every decay kind.  fp32 at head size 128 without it leaves out the
// per-dim decay, whose fp32 table of cumulative decays does not fit the LDS
// beside the fp32 tiles (the other two kinds take about 144 KB).
template <typename IT, int D, int G, bool FULL>
static void launch_dg(int dk, const DeltaArgs& a, hipStream_t st) {
  constexpr int NTH = DeltaShape<G>::NTH;
  if (dk == 0)
    hipLaunchKernelGGL((delta_kernel<IT, D, G, 0>), dim3(a.units * (a.hg_count > 0 ? a.hg_count : (a.hsplit > 1 ? a.hsplit : 1)) * (a.nseg > 1 ? a.nseg : 1)), dim3(NTH), 0, st, a);
  else if (dk == 1 || !FULL)
    hipLaunchKernelGGL((delta_kernel<IT, D, G, 1>), dim3(a.units * (a.hg_count > 0 ? a.hg_count : (a.hsplit > 1 ? a.hsplit : 1)) * (a.nseg > 1 ? a.nseg : 1)), dim3(NTH), 0, st, a);
  else if constexpr (FULL)
    hipLaunchKernelGGL((delta_kernel<IT, D, G, 2>), dim3(a.units * (a.hg_count > 0 ? a.hg_count : (a.hsplit > 1 ? a.hsplit : 1)) * (a.nseg > 1 ? a.nseg : 1)), dim3(NTH), 0, st, a);
}

template <typename IT, int D, bool FULL>
static void launch_dd(int dk, int G, const DeltaArgs& a, hipStream_t st) {
  switch (G) {
    case 1: launch_dg<IT, D, 1, FULL>(dk, a, st); break;
    case 2: launch_dg<IT, D, 2, FULL>(dk, a, st); break;
    case 4: launch_dg<IT, D, 4, FULL>(dk, a, st); break;
    default: launch_dg<IT, D, 8, FULL>(dk, a, st); break;
  }
}

template <typename IT>
static hipError_t launch_dt(int dk, int D, int G, const DeltaArgs& a, hipStream_t st) {
  switch (D) {
    case 32: launch_dd<IT, 32, true>(dk, G, a, st); break;
    case 64: launch_dd<IT, 64, true>(dk, G, a, st); break;
    default:
      if constexpr (sizeof(IT) == 2) {
        launch_dd<IT, 128, true>(dk, G, a, st);
      } else {
        if (dk == 2) return hipErrorInvalidValue;
        launch_dd<IT, 128, false>(dk, G, a, st);
      }
      break;
  }
  return hipGetLastError();
}

// start(s + 1) = M_s start(s) + N_s, one workgroup per unit, in order over the
// segments.  The running state and M_s sit in LDS (fp32); thread (ri, ci)
// forms the (D/16) x (D/16) block of rows ri * D/16 .., columns ci * D/16 ..
// of the product.
constexpr int kComposeThreads = 256;
template <int D>
__global__ __launch_bounds__(kComposeThreads) void delta_compose_kernel(const float* __restrict__ M,
                                                                     const float* __restrict__ N,
                                                                     const float* __restrict__ past,
                                                                     float* __restrict__ start, int nseg) {
  constexpr int E = D * D, RB = D / 16;
  __shared__ float Sx[E], Mx[E];
  const int tid = threadIdx.x, u = blockIdx.x;
  const int ri = tid / 16, ci = tid % 16;
  const float* pu = past ? past + (int64_t)u * E : nullptr;
  for (int i = tid; i < E; i += kComposeThreads) Sx[i] = pu ? pu[i] : 0.f;
  __syncthreads();
  for (int s = 0; s < nseg; ++s) {
    float* st = start + ((int64_t)u * nseg + s) * E;
    for (int i = tid; i < E; i += kComposeThreads) st[i] = Sx[i];
    if (s == nseg - 1) break;
    const float* ms = M + ((int64_t)u * (nseg - 1) + s) * E;
    const float* nsl = N + ((int64_t)u * (nseg - 1) + s) * E;
    for (int i = tid; i < E; i += kComposeThreads) Mx[i] = ms[i];
    __syncthreads();
    float acc[RB][RB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int c = 0; c < RB; ++c) acc[r][c] = 0.f;
    for (int k = 0; k < D; ++k) {
      float mv[RB], sv[RB];
#pragma unroll
      for (int r = 0; r < RB; ++r) mv[r] = Mx[(ri * RB + r) * D + k];
#pragma unroll
      for (int c = 0; c < RB; ++c) sv[c] = Sx[k * D + ci * RB + c];
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < RB; ++c) acc[r][c] = fmaf(mv[r], sv[c], acc[r][c]);
    }
    __syncthreads();  // every thread is done reading Sx
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int c = 0; c < RB; ++c) {
        const int i = (ri * RB + r) * D + ci * RB + c;
        Sx[i] = acc[r][c] + nsl[i];
      }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void eye_kernel(float* p, int D) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < D * D) p[i] = (i / D == i % D) ? 1.f : 0.f;
}

hipError_t launch_delta_compose(const float* M, const float* N, const float* past, float* start, int units,
                                int nseg, int D, hipStream_t st) {
  if (units <= 0) return hipSuccess;
  if (D == 32)
    hipLaunchKernelGGL(delta_compose_kernel<32>, dim3(units), dim3(kComposeThreads), 0, st, M, N, past, start, nseg);
  else if (D == 64)
    hipLaunchKernelGGL(delta_compose_kernel<64>, dim3(units), dim3(kComposeThreads), 0, st, M, N, past, start, nseg);
  else if (D == 128)
    hipLaunchKernelGGL(delta_compose_kernel<128>, dim3(units), dim3(kComposeThreads), 0, st, M, N, past, start, nseg);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_eye(float* p, int D, hipStream_t st) {
  hipLaunchKernelGGL(eye_kernel, dim3((D * D + kThreads - 1) / kThreads), dim3(kThreads), 0, st, p, D);
  return hipGetLastError();
}

hipError_t launch_delta(int io, int D, int G, int decay_kind, const DeltaArgs& a, hipStream_t st) {
  if (a.units <= 0) return hipSuccess;
  switch (io) {
    case kIoBF16: return launch_dt<uint16_t>(decay_kind, D, G, a, st);
    case kIoF16: return launch_dt<f16_t>(decay_kind, D, G, a, st);
    default: return launch_dt<float>(decay_kind, D, G, a, st);
  }
}

}  // namespace la
