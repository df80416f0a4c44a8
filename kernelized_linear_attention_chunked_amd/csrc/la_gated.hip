// Gated linear recurrence with grouped-query heads, chunk-parallel (the
// "LinearAttention" operator page, ai.onnx since version 27, "gated" rule with a
// per-head scalar decay, and "linear" when there is no decay):
//   S_t = exp(g_t) S_{t-1} + k_t v_t^T ,   o_t = scale * q_t^T S_t
// Query head h of a group reads kv head h / G.  The page allows any
// chunk-parallel evaluation that reproduces the sequential recurrence.
//
// Inside a chunk of 64 tokens, with b_i = sum_{s<=i} g_s (inclusive, per chunk):
//   o_i = scale * [ exp(b_i) q_i^T S_prev + sum_{j<=i} exp(b_i - b_j) (q_i.k_j) v_j ]
//   S   = exp(b_63) S_prev + sum_j exp(b_63 - b_j) k_j v_j^T
// Every factor is exp of a sum of g over a later stretch of tokens, so for
// g <= 0 it never exceeds 1 (exp(-b_j) alone is never formed).
//
// The output scale multiplies exp(b_i) and the exp(b_i - b_j) factors.
//
// One workgroup serves one (batch, kv head) unit and a segment of chunks, with
// all G query heads of the group: 4*P wavefronts, wave w = (head part hp =
// w/4, row part wr = w%4, reversed for w >= 4); the wave owns query rows
// [16wr, 16wr+16) of heads
// hp, hp+P, ...  The state tiles are spread over all waves.  The k/v/decay of
// a chunk are loaded once and shared by the G heads.
#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

template <int G>
struct GatedShape {
  static constexpr int P = G >= 2 ? 2 : 1;  // head parts per workgroup
  static constexpr int NW = 4 * P;          // wavefronts
  static constexpr int NTH = 64 * NW;       // threads
  static constexpr int HPW = G / P;         // query heads per wave
};

// The second bound is the minimum number of waves per SIMD: the bf16 state pass
// of an 8-wave workgroup is held to 128 registers (two workgroups per CU).
template <typename DT, int G, int MODE>
struct GatedOccupancy {
  static constexpr int value = (GatedShape<G>::NW == 8 && MODE != kModeCausal && sizeof(DT) == 2) ? 4 : 1;
};

// IT: the I/O element type (Io<IT>); DT: the operand type it is computed in.
template <typename IT, int D, int G, int MODE>
__global__ __launch_bounds__(GatedShape<G>::NTH, (GatedOccupancy<IT, G, MODE>::value)) void gated_kernel(GatedArgs a) {
  using DT = typename Io<IT>::DT;
  using O = Op<DT>;
  using SH = GatedShape<G>;
  constexpr int P = SH::P, NW = SH::NW, NTH = SH::NTH, HPW = SH::HPW;
  constexpr int VEC = O::VEC, KB = O::KB, ESZ = O::ESZ;
  constexpr int NDT = D / 16;
  constexpr int CB = D / VEC;
  // loading threads; bf16 V^T writes pack token pairs, so at least 2 tokens each
  constexpr int LOADERS = (kChunk * CB / NTH >= 2 || ESZ == 4) ? (NTH < kChunk * CB ? NTH : kChunk * CB)
                                                                : kChunk * CB / 2;
  constexpr int NTOK = kChunk * CB / LOADERS;
  constexpr int NQ = D / KB;
  constexpr int NKS = kChunk / KB;
  constexpr int PADE = 16 / ESZ;
  constexpr int KN_LD = D + PADE;
  constexpr int VT_LD = kChunk;
  constexpr int SB_LD = D + PADE;
  constexpr bool OUT = MODE == kModeCausal;
  // fp16 inputs: q and k stay fp16 for A = q k^T (an fp16 MFMA: exact products)
  // and k is read exactly by the state update; V is staged as hi + lo bf16
  // tiles (every fp16 value is the exact sum of two bf16 values) and each
  // product with V takes one more MFMA with the lo tile.  Only the inter-chunk
  // product q S rounds q to bf16, as S itself is.
  constexpr bool VLO = !std::is_same_v<IT, DT>;
  // lane indices re-derived per chunk and head where that removes spills:
  // elsewhere it measured slower
  // bf16 outputs with two heads per wave: by head pairs
  constexpr bool PAIR = OUT && ESZ == 2 && !VLO && GatedShape<G>::HPW == 2;
  constexpr bool REFRESH = PAIR || (D >= 128 && (G == 8 || (VLO && G >= 2) || (ESZ == 4 && G >= 4) || !OUT));
  constexpr int KN_BYTES = kChunk * KN_LD * ESZ;
  constexpr int VT_BYTES = D * VT_LD * ESZ;
  constexpr int VL_BYTES = VLO ? D * VT_LD * ESZ : 0;
  constexpr int SB_BYTES = OUT ? D * SB_LD * ESZ : 0;
  // per-wave 16-row tiles through which q comes in and the outputs go out as
  // whole rows (the MFMA layouts alone touch 16 rows per instruction), where
  // LDS allows
  constexpr int IO_BYTES_ = OUT ? NW * 16 * SB_LD * ESZ : 0;
  constexpr bool STAGE_IO = OUT && (KN_BYTES + VT_BYTES + SB_BYTES + VL_BYTES + IO_BYTES_ + 16 <= 160 * 1024);
  constexpr int IO_BYTES = STAGE_IO ? IO_BYTES_ : 0;
  constexpr int NS = NDT * NDT;
  constexpr int TPW = (NS + NW - 1) / NW;
  static_assert(NTOK >= 1 && NQ >= 1, "unsupported head size");
  static_assert(ESZ == 4 || NTOK % 2 == 0, "bf16 V^T writes pack token pairs");

  __shared__ __align__(16) unsigned char smem[KN_BYTES + VT_BYTES + SB_BYTES + IO_BYTES + VL_BYTES + 16];
  DT* Kn = (DT*)smem;  // k as loaded (bf16 or fp32 operands, or raw fp16)
  DT* Vt = (DT*)(smem + KN_BYTES);
  DT* Sb = (DT*)(smem + KN_BYTES + VT_BYTES);
  DT* IoT = (DT*)(smem + KN_BYTES + VT_BYTES + SB_BYTES);
  DT* Vl = (DT*)(smem + KN_BYTES + VT_BYTES + SB_BYTES + IO_BYTES);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves w and w + 4 share a SIMD: row blocks wr and 3 - wr even out the
  // causal work between SIMDs
  const int hp = w >> 2, wr = (w & 4) ? 3 - (w & 3) : (w & 3);
  int l = tid & 63, lr = l & 15, lg = l >> 4;
  auto refresh = [&]() {
    if constexpr (REFRESH) {
      l = opaque_lane(tid);
      lr = l & 15;
      lg = l >> 4;
    }
  };
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
  // token strides of q/out, k/v and the decay.  In reversed time the bases
  // sit at row T-1 and the strides are negated, so token t (always in
  // [0, T) where it is addressed) is row T-1-t.
  const int QS0 = Hq * D, KS0 = Hkv * D;
  const bool rev = a.reverse != 0;
  const int QS = rev ? -QS0 : QS0, KS = rev ? -KS0 : KS0, GS = rev ? -Hkv : Hkv;
  const int64_t row0 = rev ? (int64_t)b * T + (T - 1) : (int64_t)b * T;  // row of token 0
  const IT* qb = (const IT*)a.q + row0 * QS0 + (int64_t)(j * G * hs + hg * G) * D;
  IT* ob = (IT*)a.out + row0 * QS0 + (int64_t)(j * G * hs + hg * G) * D;
  const IT* kb = (const IT*)a.k + row0 * KS0 + (int64_t)j * D;
  const IT* vb = (const IT*)a.v + row0 * KS0 + (int64_t)j * D;
  const IT* gb = a.decay ? (const IT*)a.decay + row0 * Hkv + j : nullptr;
  const float scale = a.scale;
  // LDS element offsets (layouts and swizzles of la_device.hpp)
  auto vt_at = [&](int r, int blk) { return r * VT_LD + ((blk ^ vt_swz(r)) * VEC); };
  auto kn_at = [&](int t, int col) {
    return t * KN_LD + (((col / VEC) ^ (kn_swz(t) & (CB - 1))) * VEC) + (col % VEC);
  };
  auto sq_at = [&](int r, int col) {
    return r * SB_LD + (((col / VEC) ^ sq_swz(r)) * VEC) + (col % VEC);
  };

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

  // ---- prefetch registers
  const int cb = tid % CB, tg = tid / CB;
  const bool loader = tid < LOADERS;
  u32x4_t pk[NTOK], pv[NTOK], pq[OUT ? HPW * NQ : 1];
  // Prefetches are unconditional loads from addresses clamped to the last token
  // (tokens past the end are zeroed when staged, or never stored), and nothing
  // reads a prefetched register before it is consumed: a select, copy or
  // conversion of a register still being loaded would make the load wait.
  uint32_t pgr = 0u;  // raw bits of the decay of token l of the chunk
  auto load_g = [&](const IT* p) -> uint32_t {
    if constexpr (ESZ == 2)
      return (uint32_t)*(const uint16_t*)p;
    else
      return *(const uint32_t*)p;
  };
  auto prefetch_kvg = [&](int c) {
    const int tb = c * kChunk;
    if (loader) {
#pragma unroll
      for (int n = 0; n < NTOK; ++n) {
        const int tok = min(tb + tg * NTOK + n, T - 1);
        const int64_t off = (int64_t)tok * KS + cb * VEC;
        pk[n] = ld16(kb + off);
        pv[n] = ld16(vb + off);
      }
    }
    // without a decay input (the plain linear rule) some valid word is read and
    // ignored, so that the load is unconditional
    pgr = load_g(gb ? gb + (int64_t)min(tb + l, T - 1) * GS : kb);
  };
  // the wave's own query rows of its heads.  Staged: whole rows (piece g = 64n + l
  // of a head's 16 x D block is row g / CB, 16-byte block g % CB), parked in the
  // wave's tile when the head is computed; else straight in operand layout.
  DT* io = IoT + w * 16 * SB_LD;
  auto prefetch_q = [&](int c) {
    if constexpr (OUT) {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const int hq = hp + P * hh;
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
          if constexpr (STAGE_IO) {
            const int g = 64 * m + l;
            const int tok = min(c * kChunk + 16 * wr + g / CB, T - 1);
            pq[hh * NQ + m] = ld16(qb + (int64_t)tok * QS + hq * D + (g % CB) * VEC);
          } else {
            const int tok = min(c * kChunk + 16 * wr + lr, T - 1);
            pq[hh * NQ + m] = ld16(qb + (int64_t)tok * QS + hq * D + KB * m + VEC * lg);
          }
        }
      }
    }
  };
  static_assert(!STAGE_IO || NQ * 64 == 16 * CB, "a head's 16 rows are NQ row-wise loads per lane");

  // V -> V^T [dv][token] (swizzled) at `base`: element e of every loaded vector
  // goes to V^T row cb*VEC + e; the thread's NTOK consecutive tokens sit side by
  // side (a thread's tokens may span several 16-byte blocks, which the swizzle
  // does not keep adjacent: each group is addressed by itself)
  auto write_vt = [&](DT* base, const u32x4_t (&src)[NTOK]) {
    const int t0 = tg * NTOK;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int r = cb * VEC + e;
      if constexpr (ESZ == 2) {
#pragma unroll
        for (int n = 0; n < NTOK; n += 2) {
          const uint32_t w0 = src[n][e >> 1], w1 = src[n + 1][e >> 1];
          // low halves of both words for even e, high halves for odd e
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

  float bcs = 0.f;  // lane l: inclusive cumulative decay of token l of the chunk
  float seg_log = 0.f;
  auto stage = [&](int c) {
    const int tb = c * kChunk;
    if (tb + kChunk > T && loader) {
      // ragged last chunk: tokens past the end contribute nothing
#pragma unroll
      for (int n = 0; n < NTOK; ++n)
        if (tb + tg * NTOK + n >= T) {
          pk[n] = u32x4_t{0u, 0u, 0u, 0u};
          pv[n] = u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    if (loader) {
#pragma unroll
      for (int n = 0; n < NTOK; ++n) st16(Kn + kn_at(tg * NTOK + n, cb * VEC), pk[n]);
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
    }
    // inclusive scan of the chunk's decays across the wave (each wave keeps its own copy)
    float x = (gb && tb + l < T) ? Io<IT>::to_f32(pgr) : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off);
      if (l >= off) x += y;
    }
    bcs = x;
  };

  auto compute = [&](int c) {
    refresh();
    // b at the chunk's last token: the end of the sequence in a partial chunk,
    // so that the newest token's factor exp(btot - b_t) is exactly 1 (the scan
    // sums the padded zeros in another order, which strong decays, |b| in the
    // hundreds, would turn into a relative error of 1e-4)
    const float btot = __shfl(bcs, min(kChunk, T - c * kChunk) - 1);
    if constexpr (OUT) {
      const float bi = __shfl(bcs, 16 * wr + lr);
      // the output scale rides on both factors, so the outputs take no multiply
      const float ebi = scale * __expf(bi);
      // A^T tiles of the wave's query block: bf16 uses two per key pair p with
      // permuted rows (element q of tile (p, odd) is key 32p + 8lg + 4odd + q,
      // so that lane group lg holds keys 32p + 8lg + (0..7): one 16-byte V^T
      // read per value tile); fp32 uses single key tiles (key 16jt + 4lg + q).
      // Each element carries the decay factor exp(b_i - b_j), 0 above the
      // diagonal.  With fp16 inputs (whose V lo tile adds to the live registers)
      // a tile is formed right before its product with V, so that few are live
      // at once; otherwise all are formed first, which schedules better.
      constexpr bool LATE_A = VLO;
      constexpr int NAT = 4;
      auto need = [&](int t) { return ESZ == 2 ? (32 * (t >> 1) <= 16 * wr + 15) : (t <= wr); };
      auto key_of = [&](int t, int q) {
        return ESZ == 2 ? 32 * (t >> 1) + 8 * lg + 4 * (t & 1) + q : 16 * t + 4 * lg + q;
      };
      // decay factor of element q of tile t (computed once per chunk, for all
      // heads, where the tiles are formed early)
      auto fac_of = [&](int t, int q) {
        const int key = key_of(t, q);
        const float bj = __shfl(bcs, key);
        return key <= 16 * wr + lr ? scale * __expf(bi - bj) : 0.f;
      };
      float fac[LATE_A ? 1 : NAT][4];
      if constexpr (!LATE_A) {
#pragma unroll
        for (int t = 0; t < NAT; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) fac[t][q] = fac_of(t, q);
      }
      const int tok = c * kChunk + 16 * wr + lr;
      if constexpr (PAIR) {
        // head pairs: each K, S^T and V^T operand is read from LDS once for
        // both heads of a pair
#pragma unroll
        for (int hh = 0; hh < HPW; hh += 2) {
          refresh();
          u32x4_t qo0[NQ], qo1[NQ];
          auto q_operands = [&](int h, u32x4_t (&qo)[NQ]) {
            if constexpr (STAGE_IO) {
#pragma unroll
              for (int m = 0; m < NQ; ++m) {
                const int g = 64 * m + l;
                st16(io + sq_at(g / CB, (g % CB) * VEC), pq[h * NQ + m]);
              }
#pragma unroll
              for (int m = 0; m < NQ; ++m) qo[m] = ld16(io + sq_at(lr, KB * m + VEC * lg));
            } else {
#pragma unroll
              for (int m = 0; m < NQ; ++m) qo[m] = pq[h * NQ + m];
            }
          };
          q_operands(hh, qo0);
          q_operands(hh + 1, qo1);
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
              const u32x4_t av = ld16(Sb + sq_at(16 * ct + lr, KB * m + VEC * lg));
              O::mma(n0[ct], av, qo0[m]);
              O::mma(n1[ct], av, qo1[m]);
            }
          }
#pragma unroll
          for (int ct = 0; ct < NDT; ++ct) {
            n0[ct] *= ebi;
            n1[ct] *= ebi;
          }
          // the decayed A^T tile t of both heads
          auto a_tiles = [&](int t, f32x4_t& at0, f32x4_t& at1) {
            at0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
            at1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const int krow = 32 * (t >> 1) + 8 * (lr >> 2) + 4 * (t & 1) + (lr & 3);
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
              const u32x4_t kv = ld16(Kn + kn_at(krow, KB * m + VEC * lg));
              O::mma(at0, kv, qo0[m]);
              O::mma(at1, kv, qo1[m]);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              at0[q] *= fac[t][q];
              at1[q] *= fac[t][q];
            }
          };
          // bf16 hi + lo B operands of a tile pair
          auto operands = [&](const f32x4_t& at0, const f32x4_t& at1, u32x4_t& bh, u32x4_t& bl) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const f32x4_t& at = (e >> 1) ? at1 : at0;
              const float x0 = at[2 * (e & 1)], x1 = at[2 * (e & 1) + 1];
              const uint32_t hw = pack_bf16x2(x0, x1);
              bh[e] = hw;
              bl[e] = pack_bf16x2(x0 - __uint_as_float(hw << 16), x1 - __uint_as_float(hw & 0xffff0000u));
            }
          };
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            if (need(2 * p)) {
              f32x4_t e0, o0, e1, o1;  // tiles 2p (even) and 2p+1 (odd) of heads 0, 1
              a_tiles(2 * p, e0, e1);
              a_tiles(2 * p + 1, o0, o1);
              u32x4_t bh0, bl0, bh1, bl1;
              operands(e0, o0, bh0, bl0);
              operands(e1, o1, bh1, bl1);
#pragma unroll
              for (int ct = 0; ct < NDT; ++ct) {
                const u32x4_t av = ld16(Vt + vt_at(16 * ct + lr, 4 * p + lg));
                O::mma(n0[ct], av, bh0);
                O::mma(n1[ct], av, bh1);
                O::mma(n0[ct], av, bl0);
                O::mma(n1[ct], av, bl1);
              }
            }
          }
          auto put = [&](int h, const f32x4_t (&n)[NDT]) {
            if constexpr (STAGE_IO) {
#pragma unroll
              for (int ct = 0; ct < NDT; ++ct)
                store4((IT*)(io + sq_at(lr, 16 * ct + 4 * lg)), n[ct][0], n[ct][1], n[ct][2], n[ct][3]);
#pragma unroll
              for (int m = 0; m < NQ; ++m) {
                const int g = 64 * m + l;
                const int row = c * kChunk + 16 * wr + g / CB;
                const u32x4_t v = ld16(io + sq_at(g / CB, (g % CB) * VEC));
                if (row < T) st16(ob + (int64_t)row * QS + (hp + P * h) * D + (g % CB) * VEC, v);
              }
            } else if (tok < T) {
              IT* orow = ob + (int64_t)tok * QS + (hp + P * h) * D + 4 * lg;
#pragma unroll
              for (int ct = 0; ct < NDT; ++ct)
                store4(orow + 16 * ct, n[ct][0], n[ct][1], n[ct][2], n[ct][3]);
            }
          };
          put(hh, n0);
          put(hh + 1, n1);
        }
      } else {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        refresh();
        // the head's queries in operand layout (row lr, dk KB*m + VEC*lg), as
        // loaded (raw fp16 for fp16 inputs)
        u32x4_t qop[NQ];
        if constexpr (STAGE_IO) {
#pragma unroll
          for (int m = 0; m < NQ; ++m) {
            const int g = 64 * m + l;
            st16(io + sq_at(g / CB, (g % CB) * VEC), pq[hh * NQ + m]);
          }
#pragma unroll
          for (int m = 0; m < NQ; ++m) qop[m] = ld16(io + sq_at(lr, KB * m + VEC * lg));
        } else {
#pragma unroll
          for (int m = 0; m < NQ; ++m) qop[m] = pq[hh * NQ + m];
        }
        // decayed A^T tile t (keys as above) of this head
        auto a_tile = [&](int t) {
          f32x4_t at = f32x4_t{0.f, 0.f, 0.f, 0.f};
          const int krow = ESZ == 2 ? 32 * (t >> 1) + 8 * (lr >> 2) + 4 * (t & 1) + (lr & 3) : 16 * t + lr;
#pragma unroll
          for (int m = 0; m < NQ; ++m) {
            const u32x4_t kv = ld16(Kn + kn_at(krow, KB * m + VEC * lg));
            if constexpr (VLO)
              mma_f16(at, kv, qop[m]);
            else
              O::mma(at, kv, qop[m]);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) at[q] *= LATE_A ? fac_of(t, q) : fac[LATE_A ? 0 : t][q];
          return at;
        };
        f32x4_t at_early[LATE_A ? 1 : NAT];
        if constexpr (!LATE_A) {
#pragma unroll
          for (int t = 0; t < NAT; ++t) at_early[t] = need(t) ? a_tile(t) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        // inter-chunk term first, with the exact query; lane's column is its own
        // query i, so exp(b_i) is applied per lane to the accumulators.
        f32x4_t nacc[NDT];
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) nacc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
          // (an fp16 query becomes a bf16 operand here, like S)
          const u32x4_t qb = VLO ? Io<IT>::to_operand(qop[m]) : qop[m];
#pragma unroll
          for (int ct = 0; ct < NDT; ++ct) {
            const u32x4_t av = ld16(Sb + sq_at(16 * ct + lr, KB * m + VEC * lg));
            O::mma(nacc[ct], av, qb);
          }
        }
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) nacc[ct] *= ebi;
        if constexpr (ESZ == 2) {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            if (need(2 * p)) {
              const f32x4_t at0 = LATE_A ? a_tile(2 * p) : at_early[LATE_A ? 0 : 2 * p];
              const f32x4_t at1 = LATE_A ? a_tile(2 * p + 1) : at_early[LATE_A ? 0 : 2 * p + 1];
              // the terms of A V cancel, so A carries its bf16 rounding residual too
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
              const f32x4_t at = LATE_A ? a_tile(jt) : at_early[LATE_A ? 0 : jt];
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
        if constexpr (STAGE_IO) {
          // out through the tile (after the operand reads: one wave's LDS
          // accesses stay in order), then whole rows to memory
#pragma unroll
          for (int ct = 0; ct < NDT; ++ct)
            store4((IT*)(io + sq_at(lr, 16 * ct + 4 * lg)), nacc[ct][0], nacc[ct][1], nacc[ct][2], nacc[ct][3]);
#pragma unroll
          for (int m = 0; m < NQ; ++m) {
            const int g = 64 * m + l;
            const int row = c * kChunk + 16 * wr + g / CB;
            const u32x4_t v = ld16(io + sq_at(g / CB, (g % CB) * VEC));
            if (row < T) st16(ob + (int64_t)row * QS + (hp + P * hh) * D + (g % CB) * VEC, v);
          }
        } else if (tok < T) {
          IT* orow = ob + (int64_t)tok * QS + (hp + P * hh) * D + 4 * lg;
#pragma unroll
          for (int ct = 0; ct < NDT; ++ct)
            store4(orow + 16 * ct, nacc[ct][0], nacc[ct][1], nacc[ct][2], nacc[ct][3]);
        }
      }
      }
    }
    // the heads are done with this chunk's queries: load the next chunk's (the
    // last chunk reloads itself: an unconditional load leaves nothing to merge)
    prefetch_q(min(c + 1, c1 - 1));
    // state: S = exp(btot) S + sum_t exp(btot - b_t) k_t v_t^T
    {
      const float eb = __expf(btot);
#pragma unroll
      for (int i = 0; i < TPW; ++i) sacc[i] *= eb;
      // weight of token l in the update, one exp per lane, gathered where used
      const float wl = __expf(btot - bcs);
      u32x4_t kop[NKS], kol[NKS];
      int cur_rt = -1;
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int tau = w * TPW + i;
        if (tau < NS) {
          const int rt = tau / NDT, ct = tau % NDT;
          if (rt != cur_rt) {
            cur_rt = rt;
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
              float f[VEC];
#pragma unroll
              for (int e = 0; e < VEC; ++e) {
                const int off = kn_at(KB * m + VEC * lg + e, 16 * rt + lr);
                const float kw = __shfl(wl, KB * m + VEC * lg + e);
                if constexpr (ESZ == 2)
                  f[e] = Io<IT>::to_f32(((const uint16_t*)Kn)[off]) * kw;
                else
                  f[e] = ((const float*)Kn)[off] * kw;
              }
              kop[m] = O::pack(f);
              if constexpr (ESZ == 2) {
                // decayed keys = hi + lo in bf16
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
          for (int m = 0; m < NKS; ++m) {
            const u32x4_t bv = ld16(Vt + vt_at(16 * ct + lr, (KB / VEC) * m + lg));
            O::mma(sacc[i], kop[m], bv);
            if constexpr (ESZ == 2) O::mma(sacc[i], kol[m], bv);
            if constexpr (VLO) O::mma(sacc[i], kop[m], ld16(Vl + vt_at(16 * ct + lr, (KB / VEC) * m + lg)));
          }
        }
      }
      seg_log += btot;
    }
  };

  if (c0 < c1) {
    prefetch_kvg(c0);
    prefetch_q(c0);
  }
  for (int c = c0; c < c1; ++c) {
    stage(c);
    __syncthreads();
    prefetch_kvg(min(c + 1, c1 - 1));
    compute(c);
    __syncthreads();
    if constexpr (OUT) write_sb();
  }

  float* sout = nullptr;
  if constexpr (OUT) {
    if (s == a.nseg_total - 1 && hg == 0) sout = a.s_out + u * a.s_out_u;
  } else {
    sout = a.s_out + u * a.s_out_u + (s + a.out_slot_off) * a.s_out_s;
    if (tid == 0) a.a_out[(int64_t)u * a.nseg_total + s + a.out_slot_off] = __expf(seg_log);
  }
  if (sout) {
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
}

// In-place affine prefix over segments: slot s (s >= 1) holds the increment of
// segment s-1 and a[s] its total decay factor on entry; on exit slot s holds
// the state before segment s:  S(0) = past (or 0),  S(s) = a[s] S(s-1) + dS(s-1).
// a[s] is one factor per slot, or with a per-key-dim decay one per slot and row
// dk of S (ws_a laid out [unit][slot][dk]).
// One thread per four consecutive elements of a row of S (one decay factor for
// all four); every load of a batch of 16 slots is issued before the batch's
// stores, so a unit takes one memory round trip per batch rather than one per
// segment (slots past the last are clamped to it and their values unused).
__global__ __launch_bounds__(kThreads) void gated_prefix_kernel(float* ws_s, const float* ws_a,
                                                                const float* s_in, int U, int nseg,
                                                                int D, int per_dim) {
  constexpr int NB = 16;
  const int64_t per = (int64_t)D * D;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)U * per / 4) return;
  const int u = (int)(idx / (per / 4));
  const int64_t e = 4 * (idx % (per / 4));
  f32x4_t* base = (f32x4_t*)(ws_s + (int64_t)u * nseg * per + e);
  const int64_t stride = per / 4;
  const float* ap = per_dim ? ws_a + (int64_t)u * nseg * D + e / D : ws_a + (int64_t)u * nseg;
  const int astride = per_dim ? D : 1;
  f32x4_t acc = s_in ? *(const f32x4_t*)(s_in + (int64_t)u * per + e) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t x[NB];
  float av[NB];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int sj = min(s0 + j, nseg - 1);
      x[j] = base[sj * stride];
      av[j] = ap[sj * astride];
    }
  };
  if (nseg > 1) load_batch(1);
  base[0] = acc;
  for (int s0 = 1; s0 < nseg; s0 += NB) {
    if (s0 > 1) load_batch(s0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (s0 + j < nseg) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(av[j], acc[i], x[j][i]);
        base[(s0 + j) * stride] = acc;
      }
    }
  }
}

template <typename IT, int D, int G>
static hipError_t launch_g(int mode, const GatedArgs& a, int grid, hipStream_t st) {
  constexpr int NTH = GatedShape<G>::NTH;
  if (mode == kModeCausal)
    hipLaunchKernelGGL((gated_kernel<IT, D, G, kModeCausal>), dim3(grid), dim3(NTH), 0, st, a);
  else
    hipLaunchKernelGGL((gated_kernel<IT, D, G, kModeState>), dim3(grid), dim3(NTH), 0, st, a);
  return hipGetLastError();
}

template <typename IT, int D>
static hipError_t launch_gd(int mode, int G, const GatedArgs& a, int grid, hipStream_t st) {
  switch (G) {
    case 1: return launch_g<IT, D, 1>(mode, a, grid, st);
    case 2: return launch_g<IT, D, 2>(mode, a, grid, st);
    case 4: return launch_g<IT, D, 4>(mode, a, grid, st);
    default: return launch_g<IT, D, 8>(mode, a, grid, st);
  }
}

template <typename IT>
static hipError_t launch_gdt(int mode, int D, int G, const GatedArgs& a, int grid, hipStream_t st) {
  switch (D) {
    case 32: return launch_gd<IT, 32>(mode, G, a, grid, st);
    case 64: return launch_gd<IT, 64>(mode, G, a, grid, st);
    default: return launch_gd<IT, 128>(mode, G, a, grid, st);
  }
}

hipError_t launch_gated(int mode, int io, int D, int G, const GatedArgs& a, int grid,
                        hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  switch (io) {
    case kIoBF16: return launch_gdt<uint16_t>(mode, D, G, a, grid, st);
    case kIoF16: return launch_gdt<f16_t>(mode, D, G, a, grid, st);
    default: return launch_gdt<float>(mode, D, G, a, grid, st);
  }
}

hipError_t launch_gated_prefix(float* ws_s, const float* ws_a, const float* s_in, int U, int nseg,
                               int D, int per_dim, hipStream_t st) {
  const int64_t n = (int64_t)U * D * D / 4;
  const int grid = (int)((n + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(gated_prefix_kernel, dim3(grid), dim3(kThreads), 0, st, ws_s, ws_a, s_in, U,
                     nseg, D, per_dim);
  return hipGetLastError();
}

}  // namespace la
